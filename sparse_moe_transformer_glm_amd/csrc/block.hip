// The pre-norm block around the GLM-5.2 feed-forward layer: RMSNorm of the
// residual stream ("Full Forward" GLM-4.5 study note, How it works: pre-norm
// blocks; the GLM-5.2 anatomy page gives the same residual topology).
#include "common.h"

namespace glm {
namespace {

// bf16 nearest-even of a double, rounded once.  Outside bf16's normal range:
// round to fp32 toward zero and mark inexact results in the last bit (round
// to odd), then to bf16; with 16 spare bits in fp32 the second rounding sees
// the true position relative to the bf16 midpoint, so the result equals a
// direct rounding.  (Finite inputs.)
__device__ inline bf16_t f64_to_bf16(double v) {
  // Values in bf16's normal range (all but zero and |v| < 2^-126 in
  // practice): round the 63-bit exponent+mantissa pattern to 7 mantissa bits,
  // nearest even, with the carry running into the exponent; then rebias.
  const uint64_t u = (uint64_t)__double_as_longlong(v);
  const uint64_t mag = u & 0x7FFFFFFFFFFFFFFFull;
  const uint32_t e = (uint32_t)(mag >> 52);
  if (e > 1023 - 127 && e < 1023 + 127) {
    const uint64_t r = (mag + 0xFFFFFFFFFFFull + ((mag >> 45) & 1ull)) >> 45;
    return (bf16_t)((uint32_t)(r - ((uint64_t)(1023 - 127) << 7)) | (uint32_t)((u >> 48) & 0x8000u));
  }
  const float f = __double2float_rz(v);
  uint32_t w = __float_as_uint(f);
  if ((double)f != v) w |= 1u;
  return f32_to_bf16(__uint_as_float(w));
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

// bf16 rows of up to NC * 2048 elements: one workgroup (4 waves) per row,
// each lane holding NC 16-byte chunks in registers, so the row is read from
// memory once.  The fp64 sum of squares is reduced in a fixed order (lane
// chunks, wave butterfly, then the 4 wave sums in order), as deterministic as
// rmsnorm_kernel, though associated differently.
template <int NC>
__global__ __launch_bounds__(256) void rmsnorm_bf16_row_kernel(const bf16_t* __restrict__ h,
                                                              const float* __restrict__ w,
                                                              bf16_t* __restrict__ out, int D,
                                                              float eps) {
  __shared__ double s_part[4];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const bf16_t* hr = h + (size_t)blockIdx.x * D;
  uint4 v[NC];
#pragma unroll
  for (int c = 0; c < NC; ++c) {
    const int d = (c * 256 + tid) * 8;
    v[c] = d < D ? *reinterpret_cast<const uint4*>(hr + d) : make_uint4(0, 0, 0, 0);
  }
  double ss = 0.0;
#pragma unroll
  for (int c = 0; c < NC; ++c) {
    const uint32_t u[4] = {v[c].x, v[c].y, v[c].z, v[c].w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const double a = __uint_as_float(u[i] << 16), b = __uint_as_float(u[i] & 0xFFFF0000u);
      ss = fma(a, a, ss);
      ss = fma(b, b, ss);
    }
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) ss += __shfl_xor(ss, off, 64);
  if (lane == 0) s_part[wave] = ss;
  __syncthreads();
  ss = ((s_part[0] + s_part[1]) + s_part[2]) + s_part[3];
  const double r = 1.0 / sqrt(ss / (double)D + (double)eps);
  bf16_t* o = out + (size_t)blockIdx.x * D;
#pragma unroll
  for (int c = 0; c < NC; ++c) {
    const int d = (c * 256 + tid) * 8;
    if (d >= D) continue;
    const float4 w0 = *reinterpret_cast<const float4*>(w + d);
    const float4 w1 = *reinterpret_cast<const float4*>(w + d + 4);
    const float ww[8] = {w0.x, w0.y, w0.z, w0.w, w1.x, w1.y, w1.z, w1.w};
    const uint32_t u[4] = {v[c].x, v[c].y, v[c].z, v[c].w};
    uint32_t q[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const double a = (double)__uint_as_float(u[i] << 16) * r * (double)ww[2 * i];
      const double b = (double)__uint_as_float(u[i] & 0xFFFF0000u) * r * (double)ww[2 * i + 1];
      q[i] = (uint32_t)f64_to_bf16(a) | ((uint32_t)f64_to_bf16(b) << 16);
    }
    *reinterpret_cast<uint4*>(o + d) = make_uint4(q[0], q[1], q[2], q[3]);
  }
}

}  // namespace

hipError_t launch_rmsnorm(const void* h, const float* w, void* out, int T, int D, float eps,
                          bool bf16, hipStream_t s) {
  if (T == 0) return hipSuccess;
  const unsigned grid = (unsigned)cdiv(T, 4);
  const bf16_t* hb = static_cast<const bf16_t*>(h);
  bf16_t* ob = static_cast<bf16_t*>(out);
  const int chunks = cdiv(D, 2048);  // 16-byte chunks per lane of a 256-lane row
  if (!bf16) rmsnorm_kernel<false><<<grid, 256, 0, s>>>(h, w, out, T, D, eps);
  else if (chunks == 1) rmsnorm_bf16_row_kernel<1><<<T, 256, 0, s>>>(hb, w, ob, D, eps);
  else if (chunks == 2) rmsnorm_bf16_row_kernel<2><<<T, 256, 0, s>>>(hb, w, ob, D, eps);
  else if (chunks == 3) rmsnorm_bf16_row_kernel<3><<<T, 256, 0, s>>>(hb, w, ob, D, eps);
  else if (chunks == 4) rmsnorm_bf16_row_kernel<4><<<T, 256, 0, s>>>(hb, w, ob, D, eps);
  else rmsnorm_kernel<true><<<grid, 256, 0, s>>>(h, w, out, T, D, eps);
  return hipGetLastError();
}

}  // namespace glm
