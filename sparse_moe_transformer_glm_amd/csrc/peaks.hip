// Hardware ceilings of the GPU, measured: the rates that the layer's roofline
// fractions are also quoted against, next to the published peaks.
//
//  * bf16 MFMA: every wave of a full grid issues v_mfma_f32_32x32x16_bf16 on
//    eight independent accumulators from registers (no memory traffic in the
//    loop).  Each wave also reads the shader clock counter (s_memtime) and the
//    constant 100 MHz counter (s_memrealtime) around its loop, so the clock the
//    chip ran at under MFMA load is measured in the same launch.
//  * fp8 MFMA: the same loop on the block-scaled v_mfma_scale_f32_32x32x64_f8f6f4
//    (E4M3 operands, unit scales), the instruction of the MXFP8 layer.
//  * HBM read: a streaming read of a buffer far larger than the last-level
//    cache (16-byte non-temporal loads, one sum per thread so the loads are
//    not removed), the way the grouped GEMMs stream expert weights.
//
// Separate library (libglm_peaks.so): measurement only, not part of the layer.
#include <hip/hip_runtime.h>

#include "glm_peaks.h"

#include <stddef.h>
#include <stdint.h>

#define GLM_PEAKS_API extern "C" __attribute__((visibility("default")))

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef int i32x8 __attribute__((ext_vector_type(8)));

constexpr int kChains = 8;  // independent accumulators per wave

__global__ __launch_bounds__(256) void mfma_loop_kernel(int iters, float seed, float* sink,
                                                        unsigned long long* clocks) {
  bf16x8 a, b;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    a[i] = (__bf16)(seed + 0.001f * (threadIdx.x + i));
    b[i] = (__bf16)(seed - 0.002f * i);
  }
  f32x16 acc[kChains];
#pragma unroll
  for (int c = 0; c < kChains; ++c) acc[c] = f32x16{};
  const unsigned long long t0 = __builtin_amdgcn_s_memtime();
  const unsigned long long r0 = __builtin_amdgcn_s_memrealtime();
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int c = 0; c < kChains; ++c)
      acc[c] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc[c], 0, 0, 0);
  }
  const unsigned long long t1 = __builtin_amdgcn_s_memtime();
  const unsigned long long r1 = __builtin_amdgcn_s_memrealtime();
  float s = 0.f;
#pragma unroll
  for (int c = 0; c < kChains; ++c)
#pragma unroll
    for (int i = 0; i < 16; ++i) s += acc[c][i];
  if (s == 1.2345e30f) sink[blockIdx.x * blockDim.x + threadIdx.x] = s;  // keeps the loop
  if (threadIdx.x == 0 && blockIdx.x == 0) {
    clocks[0] = t1 - t0;
    clocks[1] = r1 - r0;
  }
}

__global__ __launch_bounds__(256) void mfma_fp8_loop_kernel(int iters, int seed, float* sink,
                                                            unsigned long long* clocks) {
  i32x8 a, b;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    a[i] = 0x38383838 + ((seed + (int)threadIdx.x + i) & 7);  // E4M3 codes near 1.0
    b[i] = 0x30303030 + (i & 3);
  }
  f32x16 acc[kChains];
#pragma unroll
  for (int c = 0; c < kChains; ++c) acc[c] = f32x16{};
  const unsigned long long t0 = __builtin_amdgcn_s_memtime();
  const unsigned long long r0 = __builtin_amdgcn_s_memrealtime();
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int c = 0; c < kChains; ++c)  // E8M0 scale 127 = 2^0
      acc[c] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, acc[c], 0, 0, 0, 127, 0,
                                                               127);
  }
  const unsigned long long t1 = __builtin_amdgcn_s_memtime();
  const unsigned long long r1 = __builtin_amdgcn_s_memrealtime();
  float s = 0.f;
#pragma unroll
  for (int c = 0; c < kChains; ++c)
#pragma unroll
    for (int i = 0; i < 16; ++i) s += acc[c][i];
  if (s == 1.2345e30f) sink[blockIdx.x * blockDim.x + threadIdx.x] = s;
  if (threadIdx.x == 0 && blockIdx.x == 0) {
    clocks[0] = t1 - t0;
    clocks[1] = r1 - r0;
  }
}

__global__ __launch_bounds__(256) void stream_read_kernel(const u32x4* __restrict__ src,
                                                          size_t n16, uint32_t* sink) {
  const size_t stride = (size_t)gridDim.x * blockDim.x;
  uint32_t acc = 0;
  size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  for (; i + 3 * stride < n16; i += 4 * stride) {
    const u32x4 v0 = __builtin_nontemporal_load(src + i);
    const u32x4 v1 = __builtin_nontemporal_load(src + i + stride);
    const u32x4 v2 = __builtin_nontemporal_load(src + i + 2 * stride);
    const u32x4 v3 = __builtin_nontemporal_load(src + i + 3 * stride);
    acc ^= v0.x ^ v0.y ^ v0.z ^ v0.w ^ v1.x ^ v1.y ^ v1.z ^ v1.w ^ v2.x ^ v2.y ^ v2.z ^ v2.w ^
           v3.x ^ v3.y ^ v3.z ^ v3.w;
  }
  for (; i < n16; i += stride) {
    const u32x4 v = __builtin_nontemporal_load(src + i);
    acc ^= v.x ^ v.y ^ v.z ^ v.w;
  }
  if (acc == 0x9E3779B9u) sink[blockIdx.x * blockDim.x + threadIdx.x] = acc;  // keeps the loads
}

int num_cus() {
  int dev = 0, cus = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
    return 0;
  return cus;
}

}  // namespace

// MFMA throughput: `blocks_per_cu` workgroups of 4 waves per compute unit,
// each wave issuing `iters` x 8 independent MFMAs: v_mfma_f32_32x32x16_bf16
// (fp8 = 0) or v_mfma_scale_f32_32x32x64_f8f6f4 (fp8 = 1).  Writes the kernel
// time (HIP events, ms), the flops performed and the shader clock observed by
// one wave (MHz: s_memtime ticks per 100 MHz s_memrealtime tick x 100).
// `scratch` is a device buffer of at least blocks * 256 floats + 16 bytes,
// owned by the caller.  Returns a hipError_t value (0 on success).
GLM_PEAKS_API int glm_peak_mfma(int fp8, int iters, int blocks_per_cu, void* scratch, float* ms,
                                double* flops, double* clock_mhz, hipStream_t stream) {
  const int cus = num_cus();
  if (cus <= 0 || iters <= 0 || blocks_per_cu <= 0 || !scratch || !ms || !flops || !clock_mhz)
    return hipErrorInvalidValue;
  const int blocks = cus * blocks_per_cu;
  unsigned long long* clocks = static_cast<unsigned long long*>(scratch);
  float* sink = reinterpret_cast<float*>(clocks + 2);
  hipEvent_t e0, e1;
  hipError_t r;
  if ((r = hipEventCreate(&e0)) != hipSuccess) return r;
  if ((r = hipEventCreate(&e1)) != hipSuccess) return r;
  auto launch = [&](int n) {
    if (fp8) mfma_fp8_loop_kernel<<<blocks, 256, 0, stream>>>(n, 1, sink, clocks);
    else mfma_loop_kernel<<<blocks, 256, 0, stream>>>(n, 0.5f, sink, clocks);
  };
  launch(iters / 8 + 1);  // warm-up
  (void)hipEventRecord(e0, stream);
  launch(iters);
  (void)hipEventRecord(e1, stream);
  if ((r = hipEventSynchronize(e1)) == hipSuccess) r = hipEventElapsedTime(ms, e0, e1);
  unsigned long long host_clocks[2] = {0, 0};
  if (r == hipSuccess) r = hipMemcpy(host_clocks, clocks, sizeof host_clocks, hipMemcpyDeviceToHost);
  (void)hipEventDestroy(e0);
  (void)hipEventDestroy(e1);
  if (r != hipSuccess) return r;
  *flops = (double)blocks * 4 * iters * kChains * (32.0 * 32 * (fp8 ? 64 : 16) * 2);
  *clock_mhz = host_clocks[1] ? 100.0 * (double)host_clocks[0] / (double)host_clocks[1] : 0.0;
  return hipSuccess;
}

// Streaming read of `bytes` (a multiple of 16) from `src` (device memory, at
// least 16-byte aligned), timed with HIP events: writes the best of `reps`
// launches in ms.  `scratch` holds at least 2048 * 256 * 4 bytes.
GLM_PEAKS_API int glm_peak_hbm_read(const void* src, size_t bytes, int reps, void* scratch,
                                    float* ms, hipStream_t stream) {
  const int cus = num_cus();
  if (cus <= 0 || !src || !scratch || !ms || bytes % 16 || reps <= 0) return hipErrorInvalidValue;
  const int blocks = cus * 8 > 2048 ? 2048 : cus * 8;
  hipEvent_t e0, e1;
  hipError_t r;
  if ((r = hipEventCreate(&e0)) != hipSuccess) return r;
  if ((r = hipEventCreate(&e1)) != hipSuccess) return r;
  const u32x4* p = static_cast<const u32x4*>(src);
  uint32_t* sink = static_cast<uint32_t*>(scratch);
  stream_read_kernel<<<blocks, 256, 0, stream>>>(p, bytes / 16, sink);  // warm-up
  float best = 1e30f;
  for (int i = 0; i < reps && r == hipSuccess; ++i) {
    (void)hipEventRecord(e0, stream);
    stream_read_kernel<<<blocks, 256, 0, stream>>>(p, bytes / 16, sink);
    (void)hipEventRecord(e1, stream);
    float t = 0.f;
    if ((r = hipEventSynchronize(e1)) == hipSuccess) r = hipEventElapsedTime(&t, e0, e1);
    if (r == hipSuccess && t < best) best = t;
  }
  (void)hipEventDestroy(e0);
  (void)hipEventDestroy(e1);
  if (r != hipSuccess) return r;
  *ms = best;
  return hipSuccess;
}
