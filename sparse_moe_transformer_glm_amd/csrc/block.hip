// The pre-norm block around the GLM-5.2 feed-forward layer: RMSNorm of the
// residual stream ("Full Forward" GLM-4.5 study note, How it works: pre-norm
// blocks; the GLM-5.2 anatomy page gives the same residual topology).
#include "common.h"

namespace glm {
namespace {

// bf16 nearest-even of a double, rounded once: round to fp32 toward zero and
// mark inexact results in the last bit (round to odd), then to bf16.  With 16
// spare bits in fp32 the second rounding sees the true position relative to
// the bf16 midpoint, so the result equals a direct rounding.  (Finite inputs.)
__device__ inline bf16_t f64_to_bf16(double v) {
  const float f = __double2float_rz(v);
  uint32_t u = __float_as_uint(f);
  if ((double)f != v) u |= 1u;
  return f32_to_bf16(__uint_as_float(u));
}

// xn[t] = h[t] / sqrt(mean(h[t]^2) + eps) * w, one wave per row.
// Arithmetic is fp64 (exact products of the bf16/fp32 inputs, fp64 sum in a
// fixed order: lane strides, then a butterfly) and the value is rounded once
// to the activation dtype.  fp32 arithmetic would move about one in 10^4
// bf16 roundings to the neighbouring value; in fp64 the rounding of every
// element is that of the exact normalised value.
template <bool BF16>
__global__ __launch_bounds__(256) void rmsnorm_kernel(const void* __restrict__ h_,
                                                      const float* __restrict__ w,
                                                      void* __restrict__ out_, int T, int D,
                                                      float eps) {
  const int lane = threadIdx.x & 63;
  const int row = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= T) return;
  double ss = 0.0;
  if constexpr (BF16) {
    const bf16_t* h = static_cast<const bf16_t*>(h_) + (size_t)row * D;
    for (int d = lane * 8; d < D; d += 64 * 8) {
      const uint4 v = *reinterpret_cast<const uint4*>(h + d);
      const uint32_t u[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const double a = __uint_as_float(u[i] << 16), b = __uint_as_float(u[i] & 0xFFFF0000u);
        ss = fma(a, a, ss);
        ss = fma(b, b, ss);
      }
    }
  } else {
    const float* h = static_cast<const float*>(h_) + (size_t)row * D;
    for (int d = lane; d < D; d += 64) ss = fma((double)h[d], (double)h[d], ss);
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) ss += __shfl_xor(ss, off, 64);
  const double r = 1.0 / sqrt(ss / (double)D + (double)eps);
  if constexpr (BF16) {
    const bf16_t* h = static_cast<const bf16_t*>(h_) + (size_t)row * D;
    bf16_t* o = static_cast<bf16_t*>(out_) + (size_t)row * D;
    for (int d = lane * 8; d < D; d += 64 * 8) {
      const uint4 v = *reinterpret_cast<const uint4*>(h + d);
      const uint32_t u[4] = {v.x, v.y, v.z, v.w};
      uint32_t q[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const double a = (double)__uint_as_float(u[i] << 16) * r * (double)w[d + 2 * i];
        const double b = (double)__uint_as_float(u[i] & 0xFFFF0000u) * r * (double)w[d + 2 * i + 1];
        q[i] = (uint32_t)f64_to_bf16(a) | ((uint32_t)f64_to_bf16(b) << 16);
      }
      *reinterpret_cast<uint4*>(o + d) = make_uint4(q[0], q[1], q[2], q[3]);
    }
  } else {
    const float* h = static_cast<const float*>(h_) + (size_t)row * D;
    float* o = static_cast<float*>(out_) + (size_t)row * D;
    for (int d = lane; d < D; d += 64) o[d] = (float)((double)h[d] * r * (double)w[d]);
  }
}

}  // namespace

hipError_t launch_rmsnorm(const void* h, const float* w, void* out, int T, int D, float eps,
                          bool bf16, hipStream_t s) {
  if (T == 0) return hipSuccess;
  const unsigned grid = (unsigned)cdiv(T, 4);
  if (bf16) rmsnorm_kernel<true><<<grid, 256, 0, s>>>(h, w, out, T, D, eps);
  else rmsnorm_kernel<false><<<grid, 256, 0, s>>>(h, w, out, T, D, eps);
  return hipGetLastError();
}

}  // namespace glm
