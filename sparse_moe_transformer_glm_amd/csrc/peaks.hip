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
//    cache (16-byte non-temporal loads, many workgroups per CU so enough
//    requests are in flight; the fastest of two launch shapes).
//  * GEMM step: the K step of the 256 x 256 bf16 prefill tile with its data in
//    L2 (one 8-wave workgroup per CU, two 64 KB LDS stages filled by 16-byte
//    LDS-DMA copies, a wait and a barrier per step, 32 MFMAs per wave on
//    fragments read from LDS), and the same step with only its MFMAs or only
//    its copies: the time the tile design needs per step when no operand
//    comes from HBM.
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
constexpr int kSinkWords = 2048 * 256;  // words of the read kernel's sink (scratch)

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

// U independent 16-byte loads in flight per thread and loop trip.
template <int U>
__global__ __launch_bounds__(256) void stream_read_kernel(const u32x4* __restrict__ src,
                                                          size_t n16, uint32_t* sink) {
  const size_t stride = (size_t)gridDim.x * blockDim.x;
  uint32_t acc = 0;
  size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  for (; i + (U - 1) * stride < n16; i += U * stride) {
    u32x4 v[U];
#pragma unroll
    for (int u = 0; u < U; ++u) v[u] = __builtin_nontemporal_load(src + i + u * stride);
#pragma unroll
    for (int u = 0; u < U; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
  }
  for (; i < n16; i += stride) {
    const u32x4 v = __builtin_nontemporal_load(src + i);
    acc ^= v.x ^ v.y ^ v.z ^ v.w;
  }
  // keeps the loads; never true for the buffers read here
  if (acc == 0x9E3779B9u) sink[(blockIdx.x * blockDim.x + threadIdx.x) % kSinkWords] = acc;
}

// One wave: every `period` ticks of the 100 MHz constant counter, lane 0
// stores (shader clock counter, constant counter) to out[2i], out[2i+1];
// stops after `ticks` or `max_samples` samples and stores the count at
// out[2 * max_samples].
__global__ __launch_bounds__(64) void clock_probe_kernel(unsigned long long ticks,
                                                         unsigned long long period,
                                                         int max_samples,
                                                         unsigned long long* out) {
  const unsigned long long r0 = __builtin_amdgcn_s_memrealtime();
  unsigned long long next = r0;
  int n = 0;
  while (n < max_samples) {
    const unsigned long long r = __builtin_amdgcn_s_memrealtime();
    if (r - r0 > ticks) break;
    if (r >= next) {
      const unsigned long long c = __builtin_amdgcn_s_memtime();
      if (threadIdx.x == 0) {
        out[2 * n] = c;
        out[2 * n + 1] = r;
      }
      ++n;
      next += period;
    }
    __builtin_amdgcn_s_sleep(8);
  }
  if (threadIdx.x == 0) out[2 * max_samples] = (unsigned long long)n;
}

typedef __attribute__((address_space(3))) void lds_void;
constexpr int kStepRows = 512;      // A and B rows of a stage (256 + 256)
constexpr int kStepK = 64;          // bf16 elements per row and step (128 bytes)
constexpr int kStepRowStride = 6144;  // elements between rows of the source (12 KB)
constexpr int kStepKCycle = 16;     // K steps before the source offset wraps (2 KB per row)
// s_waitcnt immediate: vmcnt(0), no wait on expcnt and lgkmcnt
constexpr int kVmcnt0 = (7 << 4) | (0xF << 8);

__device__ inline int step_swz(int r) { return (r & 7) ^ ((r >> 3) & 1); }

// MODE 0: MFMAs only; 1: copies only; 2: copies, fragment reads and MFMAs;
// 3: as 2 with each wave's copies of the next step spread over the step, two
// after each sub-step's first row block of MFMAs, instead of all at the
// hand-over; 4: as 3 without the fragment reads (copies and MFMAs); 5:
// fragment reads and MFMAs, no copies; 6: MFMAs with the step's 64 KB moved
// through registers instead (16-byte loads of the next step after the
// barrier, LDS writes after the MFMAs), no fragment reads.
template <int MODE>
__global__ __launch_bounds__(512) void gemm_step_kernel(const uint16_t* __restrict__ src,
                                                        int iters, float* sink,
                                                        unsigned long long* clocks) {
  constexpr int NW = 8, WN = 4, FM = 4, FN = 2, TM = 128, TN = 64, CP = 8;
  __shared__ __attribute__((aligned(1024))) uint16_t S0[kStepRows * kStepK];
  __shared__ __attribute__((aligned(1024))) uint16_t S1[kStepRows * kStepK];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  for (int i = tid; i < kStepRows * kStepK; i += 512) {
    S0[i] = (uint16_t)(0x3f80 + (i & 15));
    S1[i] = (uint16_t)(0x3f00 + (i & 7));
  }
  __syncthreads();
  // copy i of wave w: stage rows (w + 8 i) * 8 .. +8; lane l fills chunk l % 8
  const uint16_t* s[CP];
#pragma unroll
  for (int i = 0; i < CP; ++i) {
    const int r = (wave + NW * i) * 8 + lane / 8;
    s[i] = src + (size_t)r * kStepRowStride + ((lane % 8) ^ step_swz(r)) * 8;
  }
  // copies [i0, i1) of this wave for step kt into stage st
  auto issue_range = [&](uint16_t* st, int kt, int i0, int i1) {
#pragma unroll
    for (int i = 0; i < CP; ++i)
      if (i >= i0 && i < i1)
        __builtin_amdgcn_global_load_lds((const void*)(s[i] + (kt % kStepKCycle) * kStepK),
                                         (lds_void*)(st + (wave + NW * i) * (8 * kStepK)), 16, 0,
                                         0);
  };
  auto issue = [&](uint16_t* st, int kt) { issue_range(st, kt, 0, CP); };
  // MODE 6: the same rows through registers
  u32x4 stg[CP];
  auto gload = [&](int kt) {
#pragma unroll
    for (int i = 0; i < CP; ++i)
      stg[i] = *reinterpret_cast<const u32x4*>(s[i] + (kt % kStepKCycle) * kStepK);
  };
  auto lwrite = [&](uint16_t* st) {
#pragma unroll
    for (int i = 0; i < CP; ++i)
      *reinterpret_cast<u32x4*>(st + (wave + NW * i) * (8 * kStepK) + lane * 8) = stg[i];
  };
  const int wm = wave / WN, wn = wave % WN;
  const int lr = lane % 32, lk = lane / 32, sw = step_swz(lr);
  f32x16 acc[FM][FN];
#pragma unroll
  for (int m = 0; m < FM; ++m)
#pragma unroll
    for (int n = 0; n < FN; ++n) acc[m][n] = f32x16{};
  bf16x8 fa[2][FM], fb[2][FN];
  auto load = [&](const uint16_t* st, int sub, int sl) {
    const int off = ((2 * sub + lk) ^ sw) * 8;
    const uint16_t* pa = st + (wm * TM + lr) * kStepK + off;
    const uint16_t* pb = st + (256 + wn * TN + lr) * kStepK + off;
#pragma unroll
    for (int n = 0; n < FN; ++n) fb[sl][n] = *reinterpret_cast<const bf16x8*>(pb + n * 32 * kStepK);
#pragma unroll
    for (int m = 0; m < FM; ++m) fa[sl][m] = *reinterpret_cast<const bf16x8*>(pa + m * 32 * kStepK);
  };
  if (MODE != 0 && MODE != 5 && MODE != 6) issue(S0, 0);
  if (MODE == 6) {
    gload(0);
    lwrite(S0);
  }
  load(S0, 0, 0);
  load(S0, 1, 1);
  const unsigned long long t0 = __builtin_amdgcn_s_memtime();
  const unsigned long long r0 = __builtin_amdgcn_s_memrealtime();
  for (int kt = 0; kt < iters; kt += 2) {
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      uint16_t* cur = h ? S1 : S0;
      uint16_t* nxt = h ? S0 : S1;
      __builtin_amdgcn_s_waitcnt(kVmcnt0);  // this wave's copies of this step
      asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
      if (MODE == 1 || MODE == 2) issue(nxt, kt + h + 1);
      if (MODE == 6) gload(kt + h + 1);
#pragma unroll
      for (int sub = 0; sub < 4; ++sub) {
        if (MODE == 2 || MODE == 3 || MODE == 5) load(cur, (sub + 1) & 3, (sub + 1) & 1);
        __builtin_amdgcn_sched_barrier(0);
        if (MODE != 1) {
#pragma unroll
          for (int m = 0; m < FM; ++m) {
#pragma unroll
            for (int n = 0; n < FN; ++n)
              acc[m][n] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[sub & 1][m], fb[sub & 1][n],
                                                                  acc[m][n], 0, 0, 0);
            if ((MODE == 3 || MODE == 4) && m == 0) {
              __builtin_amdgcn_sched_barrier(0);
              issue_range(nxt, kt + h + 1, sub * (CP / 4), (sub + 1) * (CP / 4));
              __builtin_amdgcn_sched_barrier(0);
            }
          }
        }
      }
      if (MODE == 6) {
        __builtin_amdgcn_sched_barrier(0);
        lwrite(nxt);
      }
    }
  }
  __builtin_amdgcn_s_waitcnt(kVmcnt0);
  const unsigned long long t1 = __builtin_amdgcn_s_memtime();
  const unsigned long long r1 = __builtin_amdgcn_s_memrealtime();
  float sum = 0.f;
#pragma unroll
  for (int m = 0; m < FM; ++m)
#pragma unroll
    for (int n = 0; n < FN; ++n)
#pragma unroll
      for (int i = 0; i < 16; ++i) sum += acc[m][n][i];
  sum += (float)S0[tid * 8] + (float)S1[tid * 8];
  if (sum == 1.2345e30f) sink[blockIdx.x * 512 + tid] = sum;  // keeps the work
  if (blockIdx.x == 0 && tid == 0) {
    clocks[0] = t1 - t0;
    clocks[1] = r1 - r0;
  }
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
// launches of each of two launch shapes (32 workgroups per CU with 8 loads in
// flight per thread, 64 with 4) in ms.  `scratch` holds at least
// 2048 * 256 * 4 bytes.
GLM_PEAKS_API int glm_peak_hbm_read(const void* src, size_t bytes, int reps, void* scratch,
                                    float* ms, hipStream_t stream) {
  const int cus = num_cus();
  if (cus <= 0 || !src || !scratch || !ms || bytes % 16 || reps <= 0) return hipErrorInvalidValue;
  hipEvent_t e0, e1;
  hipError_t r;
  if ((r = hipEventCreate(&e0)) != hipSuccess) return r;
  if ((r = hipEventCreate(&e1)) != hipSuccess) return r;
  const u32x4* p = static_cast<const u32x4*>(src);
  uint32_t* sink = static_cast<uint32_t*>(scratch);
  const size_t n16 = bytes / 16;
  auto launch = [&](int shape) {
    if (shape == 0) stream_read_kernel<8><<<cus * 32, 256, 0, stream>>>(p, n16, sink);
    else stream_read_kernel<4><<<cus * 64, 256, 0, stream>>>(p, n16, sink);
  };
  float best = 1e30f;
  for (int shape = 0; shape < 2 && r == hipSuccess; ++shape) {
    launch(shape);  // warm-up
    for (int i = 0; i < reps && r == hipSuccess; ++i) {
      (void)hipEventRecord(e0, stream);
      launch(shape);
      (void)hipEventRecord(e1, stream);
      float t = 0.f;
      if ((r = hipEventSynchronize(e1)) == hipSuccess) r = hipEventElapsedTime(&t, e0, e1);
      if (r == hipSuccess && t < best) best = t;
    }
  }
  (void)hipEventDestroy(e0);
  (void)hipEventDestroy(e1);
  if (r != hipSuccess) return r;
  *ms = best;
  return hipSuccess;
}

// Shader clock while other work runs: launches one wave on `stream` that
// samples the shader clock counter against the 100 MHz constant counter every
// `period_us` microseconds for `seconds` (at most 10) or `max_samples`
// samples, and returns without waiting.  `buf`: caller-owned device buffer of
// 2 * max_samples + 1 unsigned 64-bit words (pairs, then the count), valid
// once the stream has passed the probe.  A SIMD holding the probe wave may
// not fit a workgroup that needs its whole register file.
GLM_PEAKS_API int glm_peak_clock_probe(double seconds, int period_us, int max_samples, void* buf,
                                       hipStream_t stream) {
  if (!(seconds > 0.0) || seconds > 10.0 || period_us <= 0 || max_samples <= 0 || !buf)
    return hipErrorInvalidValue;
  const unsigned long long ticks = (unsigned long long)(seconds * 1e8);
  clock_probe_kernel<<<1, 64, 0, stream>>>(ticks, (unsigned long long)period_us * 100,
                                           max_samples, static_cast<unsigned long long*>(buf));
  return hipGetLastError();
}

// The K step of the 256 x 256 bf16 prefill tile with its operands in L2: one
// 8-wave workgroup per CU runs `iters` steps (even) of `mode` (0: the 32
// MFMAs per wave only; 1: only the 64 KB of LDS-DMA copies per workgroup,
// with the wait and barrier of each step; 2: copies, fragment reads and
// MFMAs; 3: as 2 with each wave's copies spread over the step, two after
// each sub-step's first row block of MFMAs; 4: as 3 without the fragment
// reads; 5: fragment reads and MFMAs without copies; 6: MFMAs with the
// rows moved through registers, 16-byte loads then LDS writes, no fragment
// reads).  The copies read rows 12 KB apart from `src`, a device buffer of at
// least 512 * 12288 bytes, 2 KB of each (about 1 MB, L2-resident).  Writes
// the time per step (*us_per_step, HIP events) and the shader clock one wave
// observed (*clock_mhz).  `scratch`: device buffer of at least
// 16 + 4 * 512 * (number of compute units) bytes.  Blocks until done.
GLM_PEAKS_API int glm_peak_gemm_step(int mode, int iters, const void* src, void* scratch,
                                     double* us_per_step, double* clock_mhz, hipStream_t stream) {
  const int cus = num_cus();
  if (cus <= 0 || mode < 0 || mode > 6 || iters <= 0 || iters % 2 || !src || !scratch ||
      !us_per_step || !clock_mhz)
    return hipErrorInvalidValue;
  unsigned long long* clocks = static_cast<unsigned long long*>(scratch);
  float* sink = reinterpret_cast<float*>(clocks + 2);
  const uint16_t* p = static_cast<const uint16_t*>(src);
  auto launch = [&](int n) {
    if (mode == 0) gemm_step_kernel<0><<<cus, 512, 0, stream>>>(p, n, sink, clocks);
    else if (mode == 1) gemm_step_kernel<1><<<cus, 512, 0, stream>>>(p, n, sink, clocks);
    else if (mode == 2) gemm_step_kernel<2><<<cus, 512, 0, stream>>>(p, n, sink, clocks);
    else if (mode == 3) gemm_step_kernel<3><<<cus, 512, 0, stream>>>(p, n, sink, clocks);
    else if (mode == 4) gemm_step_kernel<4><<<cus, 512, 0, stream>>>(p, n, sink, clocks);
    else if (mode == 5) gemm_step_kernel<5><<<cus, 512, 0, stream>>>(p, n, sink, clocks);
    else gemm_step_kernel<6><<<cus, 512, 0, stream>>>(p, n, sink, clocks);
  };
  hipEvent_t e0, e1;
  hipError_t r;
  if ((r = hipEventCreate(&e0)) != hipSuccess) return r;
  if ((r = hipEventCreate(&e1)) != hipSuccess) return r;
  launch(200);  // warm-up
  (void)hipEventRecord(e0, stream);
  launch(iters);
  (void)hipEventRecord(e1, stream);
  float ms = 0.f;
  if ((r = hipEventSynchronize(e1)) == hipSuccess) r = hipEventElapsedTime(&ms, e0, e1);
  unsigned long long host_clocks[2] = {0, 0};
  if (r == hipSuccess) r = hipMemcpy(host_clocks, clocks, sizeof host_clocks, hipMemcpyDeviceToHost);
  (void)hipEventDestroy(e0);
  (void)hipEventDestroy(e1);
  if (r != hipSuccess) return r;
  *us_per_step = ms * 1e3 / iters;
  *clock_mhz = host_clocks[1] ? 100.0 * (double)host_clocks[0] / (double)host_clocks[1] : 0.0;
  return hipSuccess;
}
