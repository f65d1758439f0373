// Router of the GLM-5.2 MoE layer: sigmoid scores, bias-adjusted top-k
// selection, un-biased renormalisation and scaling (frontier-model-atlas
// "GLM-5.2 model anatomy", Feed-forward / Mixture of Experts panel).
#include "common.h"

#include <type_traits>

namespace glm {
namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// Split 8 fp32 values into three bf16 vectors with w == hi + mid + lo exactly
// (each remainder has at most 16, then 8, significant bits).
__device__ inline void split3(const float4 w0, const float4 w1, bf16x8& hi, bf16x8& mid,
                              bf16x8& lo) {
  float v[8] = {w0.x, w0.y, w0.z, w0.w, w1.x, w1.y, w1.z, w1.w};
  uint32_t h[4], m[4], l[4];
#pragma unroll
  for (int i = 0; i < 8; i += 2) {
    bf16_t hb[2], mb[2], lb[2];
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      float a = v[i + j];
      hb[j] = f32_to_bf16(a);
      float r1 = a - bf16_to_f32(hb[j]);
      mb[j] = f32_to_bf16(r1);
      float r2 = r1 - bf16_to_f32(mb[j]);
      lb[j] = f32_to_bf16(r2);
    }
    h[i / 2] = hb[0] | (uint32_t(hb[1]) << 16);
    m[i / 2] = mb[0] | (uint32_t(mb[1]) << 16);
    l[i / 2] = lb[0] | (uint32_t(lb[1]) << 16);
  }
  hi = __builtin_bit_cast(bf16x8, (u32x4){h[0], h[1], h[2], h[3]});
  mid = __builtin_bit_cast(bf16x8, (u32x4){m[0], m[1], m[2], m[3]});
  lo = __builtin_bit_cast(bf16x8, (u32x4){l[0], l[1], l[2], l[3]});
}

#ifndef GLM_ROUTER_MT
#define GLM_ROUTER_MT 8  // 16-row token blocks per workgroup on large batches
#endif
#ifndef GLM_ROUTER_ST
#define GLM_ROUTER_ST 2  // LDS stages of the large-batch tile
#endif

// One workgroup: MT*16 tokens x 64 experts over one K slice.  Wave w owns
// experts [16w, 16w+16) and every token of the tile (MT 16-row MFMA blocks).
// MFMA 16x16x32 bf16: lane l supplies row (l % 16), k-group (l / 16) of both
// operands; the accumulator holds rows 4*(l/16)+r, column l % 16.
//
// K goes in steps of 64 through a ring of ST LDS stages filled by 16-byte
// LDS-DMA loads: the x tile (bf16 rows of 128 B) and the fp32 router rows
// (256 B) are read once per workgroup and shared by its four waves.  The
// 16-byte chunks of every row are XOR-swizzled so that the 16 rows a
// fragment read touches fall on distinct banks.  Each weight is split into
// three bf16 terms right before its MFMAs (w = hi + mid + lo exactly).
template <int MT, int ST>
__global__ __launch_bounds__(256) void router_logits_bf16_kernel(
    const bf16_t* __restrict__ x, const float* __restrict__ W, float* __restrict__ partial,
    int T, int D, int E, int kchunk, uint64_t* __restrict__ masks, int n_masks) {
  constexpr int XB = MT * 16 * 128;          // x tile bytes per stage
  constexpr int WB = 64 * 256;               // router tile bytes per stage
  constexpr int X_INST = XB / 1024, W_INST = WB / 1024;  // 1-KB DMA instructions
  constexpr int IPW = (X_INST + W_INST) / 4;
  static_assert((X_INST + W_INST) % 4 == 0, "every wave issues the same number of DMAs");
  static_assert(ST == 2 || ST == 3, "ring of two or three stages");
  __shared__ __attribute__((aligned(1024))) uint8_t lds0[XB + WB];
  __shared__ __attribute__((aligned(1024))) uint8_t lds1[XB + WB];
  __shared__ __attribute__((aligned(1024))) uint8_t lds2[ST > 2 ? XB + WB : 16];

  // clear the routing masks the top-k kernel fills
  {
    const int nb = gridDim.x * gridDim.y * gridDim.z;
    const int b = (blockIdx.z * gridDim.y + blockIdx.y) * gridDim.x + blockIdx.x;
    for (int i = b * 256 + threadIdx.x; i < n_masks; i += nb * 256) masks[i] = 0ull;
  }
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int t0 = blockIdx.x * (MT * 16);
  const int e0 = blockIdx.y * 64;
  const int ks = blockIdx.z;
  const int kbeg = ks * kchunk;
  const int nk = (min(D, kbeg + kchunk) - kbeg) / 64;

  // DMA sources: instruction q = wave + 4i fills 1 KB of the stage; lane l
  // writes physical chunk l % 8 of x row 8q + l/8, or physical chunk l % 16
  // of router row 4(q - X_INST) + l/16.
  const uint8_t* src[IPW];
  int dst[IPW];
#pragma unroll
  for (int i = 0; i < IPW; ++i) {
    const int q = wave + 4 * i;
    if (q < X_INST) {
      const int r = q * 8 + lane / 8;
      const int lc = (lane % 8) ^ ((r >> 1) & 7);
      src[i] = reinterpret_cast<const uint8_t*>(x + (size_t)min(t0 + r, T - 1) * D + kbeg + lc * 8);
      dst[i] = q * 1024;
    } else {
      const int r = (q - X_INST) * 4 + lane / 16;
      const int lc = (lane % 16) ^ (r & 15);
      src[i] = reinterpret_cast<const uint8_t*>(W + (size_t)min(e0 + r, E - 1) * D + kbeg + lc * 4);
      dst[i] = XB + (q - X_INST) * 1024;
    }
  }
  auto stage_ptr = [&](int s) -> uint8_t* { return s == 0 ? lds0 : s == 1 ? lds1 : lds2; };
  auto issue = [&](uint8_t* st, int kt) {
#pragma unroll
    for (int i = 0; i < IPW; ++i) {
      const size_t step = (wave + 4 * i < X_INST) ? (size_t)kt * 128 : (size_t)kt * 256;
      __builtin_amdgcn_global_load_lds((const void*)(src[i] + step), (lds_void*)(st + dst[i]),
                                       16, 0, 0);
    }
  };

  f32x4 acc[MT];
#pragma unroll
  for (int m = 0; m < MT; ++m) acc[m] = (f32x4){0.f, 0.f, 0.f, 0.f};

  const int r16 = lane & 15, kg = lane >> 4;
  const int xsw = (r16 >> 1) & 7;  // swizzle of x rows 16m + r16
  auto compute = [&](const uint8_t* st) {
#pragma unroll
    for (int sub = 0; sub < 2; ++sub) {
      const int xc = ((4 * sub + kg) ^ xsw) * 16;
      const int wc0 = ((8 * sub + 2 * kg) ^ r16) * 16, wc1 = ((8 * sub + 2 * kg + 1) ^ r16) * 16;
      const uint8_t* wrow = st + XB + (wave * 16 + r16) * 256;
      const float4 w0 = *reinterpret_cast<const float4*>(wrow + wc0);
      const float4 w1 = *reinterpret_cast<const float4*>(wrow + wc1);
      bf16x8 a[MT];
#pragma unroll
      for (int m = 0; m < MT; ++m)
        a[m] = *reinterpret_cast<const bf16x8*>(st + (16 * m + r16) * 128 + xc);
      bf16x8 hi, mid, lo;
      split3(w0, w1, hi, mid, lo);
#pragma unroll
      for (int m = 0; m < MT; ++m) {
        acc[m] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[m], lo, acc[m], 0, 0, 0);
        acc[m] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[m], mid, acc[m], 0, 0, 0);
        acc[m] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[m], hi, acc[m], 0, 0, 0);
      }
    }
  };

  // Step kt: wait for its stage (later stages may stay in flight), meet the
  // barrier (every wave is then also done with the stage read at kt-1),
  // refill that stage ST-1 steps ahead, compute.
#pragma unroll
  for (int s = 0; s < ST - 1; ++s)
    if (s < nk) issue(stage_ptr(s), s);
  auto step = [&](auto sc, int kt) {
    constexpr int s = decltype(sc)::value;
    if (ST == 3 && kt + 1 < nk) __builtin_amdgcn_s_waitcnt(GLM_VMCNT(IPW));
    else __builtin_amdgcn_s_waitcnt(GLM_VMCNT(0));
    lds_barrier();
    if (kt + ST - 1 < nk) issue(stage_ptr((s + ST - 1) % ST), kt + ST - 1);
    compute(stage_ptr(s));
  };
  for (int kt = 0; kt < nk; kt += ST) {
    step(std::integral_constant<int, 0>{}, kt);
    if (kt + 1 < nk) step(std::integral_constant<int, 1>{}, kt + 1);
    if constexpr (ST > 2) if (kt + 2 < nk) step(std::integral_constant<int, 2>{}, kt + 2);
  }

  const int e = e0 + wave * 16 + r16;
  if (e >= E) return;
#pragma unroll
  for (int m = 0; m < MT; ++m) {
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int t = t0 + 16 * m + 4 * kg + r;
      if (t < T) partial[((size_t)ks * T + t) * E + e] = acc[m][r];
    }
  }
}

// fp32 activations: plain fp32 dot products, one thread per (token, expert).
__global__ __launch_bounds__(256) void router_logits_f32_kernel(
    const float* __restrict__ x, const float* __restrict__ W, float* __restrict__ partial,
    int T, int D, int E, uint64_t* __restrict__ masks, int n_masks) {
  const size_t i = (size_t)blockIdx.x * 256 + threadIdx.x;
  if (i < (size_t)n_masks) masks[i] = 0ull;  // T*E threads >= masks
  if (i >= (size_t)T * E) return;
  const int t = (int)(i / E), e = (int)(i % E);
  const float* xr = x + (size_t)t * D;
  const float* wr = W + (size_t)e * D;
  float acc = 0.f;
  for (int d = 0; d < D; ++d) acc = fmaf(xr[d], wr[d], acc);
  partial[i] = acc;
}

// Order-preserving map of a float to an unsigned integer (larger float, larger key).
__device__ inline uint32_t ordered_bits(float f) {
  if (f == 0.0f) f = 0.0f;  // -0 and +0 tie
  const uint32_t u = __float_as_uint(f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// Sum of the K-slice partial logits in slice order (independent loads first).
__device__ inline float sum_partials(const float* p, size_t stride, int ksplit) {
  float z = 0.f;
  int s = 0;
  for (; s + 8 <= ksplit; s += 8) {
    float v[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) v[i] = p[(size_t)(s + i) * stride];
#pragma unroll
    for (int i = 0; i < 8; ++i) z += v[i];
  }
  for (; s < ksplit; ++s) z += p[(size_t)s * stride];
  return z;
}

// One wave per token (four tokens per workgroup).  Lane l holds experts l,
// l+64, l+128, l+192.  Selection takes k rounds of a wave-wide max over 64-bit
// keys (biased score, then lower index).  Each selection also sets the token's
// bit in masks[token / 64][expert] (an OR, so the result does not depend on
// the order of the atomics); the logits kernel has zeroed the masks.
// Wave-wide maximum of 64-bit keys.
__device__ inline unsigned long long wave_max(unsigned long long v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) {
    const unsigned long long o = __shfl_xor(v, off, 64);
    v = o > v ? o : v;
  }
  return v;
}

// Group-limited routing: experts form n_group consecutive groups; a group
// scores the sum (fp32, largest first) of its group_topk best biased scores;
// the token keeps the topk_group best groups (ties: lower group) and the keys
// of experts outside them are cleared.
__device__ inline void restrict_to_groups(unsigned long long (&key)[4], const float (&beta)[4],
                                          int lane, int E, GroupRouting gr) {
  const int gsz = E / gr.n_group;
  float my_gscore = 0.f;  // lane g < n_group holds group g's score
  for (int g = 0; g < gr.n_group; ++g) {
    unsigned long long gk[4];
#pragma unroll
    for (int c = 0; c < 4; ++c) gk[c] = ((lane + 64 * c) / gsz == g) ? key[c] : 0ull;
    float sum = 0.f;
    for (int r = 0; r < gr.group_topk; ++r) {
      unsigned long long best = gk[0];
#pragma unroll
      for (int c = 1; c < 4; ++c) best = gk[c] > best ? gk[c] : best;
      best = wave_max(best);
      const int es = (int)(~(uint32_t)best);
      const int src = es & 63, cs = es >> 6;
      float mine = beta[0];
#pragma unroll
      for (int c = 1; c < 4; ++c) mine = (cs == c) ? beta[c] : mine;
      sum += __shfl(mine, src, 64);
#pragma unroll
      for (int c = 0; c < 4; ++c)
        if (lane == src && cs == c) gk[c] = 0ull;
    }
    if (lane == g) my_gscore = sum;
  }
  unsigned long long gkey = lane < gr.n_group
      ? ((unsigned long long)ordered_bits(my_gscore) << 32) | (uint32_t)(~lane) : 0ull;
  unsigned long long keep = 0ull;  // bit g: group g kept
  for (int r = 0; r < gr.topk_group; ++r) {
    const unsigned long long best = wave_max(gkey);
    const int gs = (int)(~(uint32_t)best);
    keep |= 1ull << gs;
    if (lane == gs) gkey = 0ull;
  }
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    const int e = lane + 64 * c;
    if (e < E && !((keep >> (e / gsz)) & 1ull)) key[c] = 0ull;
  }
}

__global__ __launch_bounds__(256) void router_topk_kernel(
    const float* __restrict__ partial, int ksplit, const float* __restrict__ bias,
    int T, int E, int k, float scale, GroupRouting gr, int32_t* __restrict__ idx_out,
    float* __restrict__ w_out, unsigned long long* __restrict__ masks) {
  const int lane = threadIdx.x & 63;
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= T) return;
  const size_t stride = (size_t)T * E;
  float sig[4], beta[4];
  unsigned long long key[4];
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    const int e = lane + 64 * c;
    sig[c] = 0.f;
    beta[c] = 0.f;
    key[c] = 0ull;
    if (e < E) {
      const float z = sum_partials(partial + (size_t)t * E + e, stride, ksplit);
      const float sg = 1.0f / (1.0f + expf(-z));
      sig[c] = sg;
      beta[c] = sg + bias[e];
      key[c] = ((unsigned long long)ordered_bits(beta[c]) << 32) | (uint32_t)(~e);
    }
  }
  if (gr.n_group > 1) restrict_to_groups(key, beta, lane, E, gr);
  unsigned long long* tmask = masks + (size_t)(t / kTokTile) * E;
  const unsigned long long bit = 1ull << (t % kTokTile);
  float ssum = 0.f, my_sig = 0.f;
  int my_e = -1;
  for (int j = 0; j < k; ++j) {
    unsigned long long best = key[0];
#pragma unroll
    for (int c = 1; c < 4; ++c) best = key[c] > best ? key[c] : best;
    best = wave_max(best);
    const int es = (int)(~(uint32_t)best);
    const int src = es & 63, cs = es >> 6;
    float mine = sig[0];
#pragma unroll
    for (int c = 1; c < 4; ++c) mine = (cs == c) ? sig[c] : mine;
    const float ss = __shfl(mine, src, 64);
#pragma unroll
    for (int c = 0; c < 4; ++c)
      if (lane == src && cs == c) key[c] = 0ull;
    ssum += ss;
    if (lane == j) {
      my_e = es;
      my_sig = ss;
    }
  }
  if (lane < k) {
    idx_out[(size_t)t * k + lane] = my_e;
    w_out[(size_t)t * k + lane] = (my_sig / ssum) * scale;
    atomicOr(&tmask[my_e], bit);
  }
}

}  // namespace

int router_tile_rows(int T) { return T > 64 ? GLM_ROUTER_MT * 16 : 64; }

hipError_t launch_router_logits_bf16(const bf16_t* x, const float* router_w, float* partial,
                                     int T, int D, int E, int ksplit, int kchunk,
                                     uint64_t* masks, hipStream_t s) {
  const int rows = router_tile_rows(T);
  dim3 grid(cdiv(T, rows), cdiv(E, 64), ksplit);
  const int n_masks = cdiv(T, kTokTile) * E;
  if (rows == 64)
    router_logits_bf16_kernel<4, 3><<<grid, 256, 0, s>>>(x, router_w, partial, T, D, E, kchunk,
                                                         masks, n_masks);
  else
    router_logits_bf16_kernel<GLM_ROUTER_MT, GLM_ROUTER_ST><<<grid, 256, 0, s>>>(
        x, router_w, partial, T, D, E, kchunk, masks, n_masks);
  return hipGetLastError();
}

hipError_t launch_router_logits_f32(const float* x, const float* router_w, float* partial,
                                    int T, int D, int E, uint64_t* masks, hipStream_t s) {
  const size_t n = (size_t)T * E;
  router_logits_f32_kernel<<<(unsigned)((n + 255) / 256), 256, 0, s>>>(
      x, router_w, partial, T, D, E, masks, cdiv(T, kTokTile) * E);
  return hipGetLastError();
}

hipError_t launch_router_topk(const float* partial, int ksplit, const float* corr_bias, int T,
                              int E, int k, float scale, GroupRouting gr, int32_t* topk_idx,
                              float* topk_w, uint64_t* masks, hipStream_t s) {
  router_topk_kernel<<<cdiv(T, 4), 256, 0, s>>>(partial, ksplit, corr_bias, T, E, k, scale, gr,
                                               topk_idx, topk_w,
                                               reinterpret_cast<unsigned long long*>(masks));
  return hipGetLastError();
}

}  // namespace glm
