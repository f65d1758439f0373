// fp32 expert path of the GLM-5.2 MoE layer: the same permuted data flow as
// the bf16 path (gate/up with fused SiLU gating, weighted down projection with
// un-permuted store, shared expert plus slot-ordered combine), with every
// intermediate kept in fp32.  One thread per output element, sequential fp32
// FMA over K; meant for small layers.
#include "common.h"

namespace glm {
namespace {

__device__ inline float silu(float g) { return g / (1.0f + expf(-g)); }

// expert owning permuted row r: largest e with offsets[e] <= r
__device__ inline int expert_of_row(const int32_t* offsets, int E, int r) {
  int lo = 0, hi = E - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (offsets[mid] <= r) lo = mid; else hi = mid - 1;
  }
  return lo;
}

__device__ inline float dot(const float* a, const float* b, int n) {
  float s = 0.f;
  for (int i = 0; i < n; ++i) s = fmaf(a[i], b[i], s);
  return s;
}

__global__ __launch_bounds__(256) void gateup_f32_kernel(F32Args a) {
  const int Fm = max(a.F, a.Fs);
  const size_t i = (size_t)blockIdx.x * 256 + threadIdx.x;
  const size_t A = (size_t)a.T * a.k;
  if (i >= (A + a.T) * Fm) return;
  const int r = (int)(i / Fm), h = (int)(i % Fm);
  if ((size_t)r < A) {
    if (h >= a.F) return;
    const int e = expert_of_row(a.offsets, a.E, r);
    const float* x = a.x + (size_t)(a.row_assign[r] / a.k) * a.D;
    const float g = dot(x, a.w1 + ((size_t)e * a.F + h) * a.D, a.D);
    const float u = dot(x, a.w3 + ((size_t)e * a.F + h) * a.D, a.D);
    a.H[(size_t)r * a.F + h] = silu(g) * u;
  } else {
    if (h >= a.Fs) return;
    const int t = r - (int)A;
    const float* x = a.x + (size_t)t * a.D;
    const float g = dot(x, a.sw1 + (size_t)h * a.D, a.D);
    const float u = dot(x, a.sw3 + (size_t)h * a.D, a.D);
    a.Hs[(size_t)t * a.Fs + h] = silu(g) * u;
  }
}

__global__ __launch_bounds__(256) void down_f32_kernel(F32Args a) {
  const size_t i = (size_t)blockIdx.x * 256 + threadIdx.x;
  const size_t A = (size_t)a.T * a.k;
  if (i >= A * a.D) return;
  const int r = (int)(i / a.D), d = (int)(i % a.D);
  const int e = expert_of_row(a.offsets, a.E, r);
  const float y = dot(a.H + (size_t)r * a.F, a.w2 + ((size_t)e * a.D + d) * a.F, a.F);
  const int asg = a.row_assign[r];
  a.Y[(size_t)y_row(asg, a.k) * a.D + d] = a.topk_w[asg] * y;
}

__global__ __launch_bounds__(256) void shared_combine_f32_kernel(F32Args a) {
  const size_t i = (size_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= (size_t)a.T * a.D) return;
  const int t = (int)(i / a.D), d = (int)(i % a.D);
  float v = dot(a.Hs + (size_t)t * a.Fs, a.sw2 + (size_t)d * a.Fs, a.Fs);
  for (int j = 0; j < a.k; ++j) v += a.Y[((size_t)t * (a.k + 1) + j) * a.D + d];
  if (a.residual) v += a.residual[i];
  a.out[i] = v;
}

unsigned blocks(size_t n) { return (unsigned)((n + 255) / 256); }

}  // namespace

hipError_t launch_gateup_f32(const F32Args& a, hipStream_t s) {
  const size_t n = ((size_t)a.T * a.k + a.T) * (size_t)max(a.F, a.Fs);
  gateup_f32_kernel<<<blocks(n), 256, 0, s>>>(a);
  return hipGetLastError();
}

hipError_t launch_down_f32(const F32Args& a, hipStream_t s) {
  if ((size_t)a.T * a.k * a.D == 0) return hipSuccess;
  down_f32_kernel<<<blocks((size_t)a.T * a.k * a.D), 256, 0, s>>>(a);
  return hipGetLastError();
}

hipError_t launch_shared_combine_f32(const F32Args& a, hipStream_t s) {
  shared_combine_f32_kernel<<<blocks((size_t)a.T * a.D), 256, 0, s>>>(a);
  return hipGetLastError();
}

}  // namespace glm
