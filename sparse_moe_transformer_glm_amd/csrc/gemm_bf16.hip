// Grouped expert GEMMs of the GLM-5.2 MoE layer on gfx950 bf16 MFMA.
//
// Every product here is C[M x N] = A[M x K] . B[N x K]^T with both operands
// K-contiguous: A rows are token activations (gathered) or gated hidden rows,
// B rows are weight rows (w1/w3 [F][D], w2 [D][F]).  One workgroup computes a
// BM x BN tile: K is walked in steps of 64 through double-buffered LDS tiles
// (rows padded by 16 bytes so the MFMA fragment reads are conflict-free), and
// each wave accumulates a (BM/WM) x (BN/WN) sub-tile with
// v_mfma_f32_16x16x32_bf16.
//
// Three epilogues:
//  * GATE_UP: B-tile rows alternate 16 rows of w1 (gate) and the matching 16
//    rows of w3 (up), so one lane holds gate and up of the same hidden unit and
//    writes H = bf16(SiLU(g) * u)  (SiLU-gated expert MLP; w1/w3/w2 roles as on
//    the PocketLLM "GLM-5.2" page, Implemented execution path).
//  * DOWN: Y[t*k+j] = w[t][j] * (H W2^T): the routing weight is applied and the
//    row is written straight to its (token, slot) place (un-permute); no atomics.
//  * SHARED_COMBINE: out[t] = Hs[t] Ws2^T + sum_j Y[t*k+j] in slot order: the
//    always-on shared expert merged with the weighted routed outputs
//    (GLM-5.2 anatomy page, Mixture of Experts panel).
#include "common.h"

namespace glm {
namespace {

enum Mode { GATE_UP = 0, DOWN = 1, SHARED_COMBINE = 2 };

constexpr int BK = 64;          // K step (bf16 elements) = 8 chunks of 16 bytes
constexpr int LDK = BK + 8;     // padded LDS row (elements)

template <int BM, int BN, int WM, int WN>
struct Tile {
  static constexpr int NT = WM * WN * kWave;
  static constexpr int TM = BM / WM, TN = BN / WN;
  static constexpr int FM = TM / 16, FN = TN / 16;
  static constexpr int A_CHUNKS = BM * (BK / 8), B_CHUNKS = BN * (BK / 8);
  static constexpr int A_PER = (A_CHUNKS + NT - 1) / NT;
  static constexpr int B_PER = (B_CHUNKS + NT - 1) / NT;
  static_assert(TM % 16 == 0 && TN % 16 == 0, "wave tile must be a multiple of 16");
};

__device__ inline float silu(float g) { return g / (1.0f + expf(-g)); }

// Maps a workgroup to a logical tile index.  Logical tiles are split into 8
// contiguous chunks, one per XCD (workgroups are dispatched round-robin over
// the XCDs), so tiles that share a weight slice or an activation block run on
// the same XCD and share its L2.
__device__ inline int xcd_tile(int n) {
  const int c = (n + kXcds - 1) / kXcds;
  const int x = blockIdx.x % kXcds, o = blockIdx.x / kXcds;
  if (o >= c) return -1;
  const int i = x * c + o;
  return i < n ? i : -1;
}

template <int BM, int BN, int WM, int WN, int MODE>
__global__ __launch_bounds__(WM* WN* kWave) void grouped_gemm_kernel(GateUpArgs gu, DownArgs dn,
                                                                    CombineArgs cb) {
  using Tl = Tile<BM, BN, WM, WN>;
  constexpr int NT = Tl::NT, FM = Tl::FM, FN = Tl::FN, TM = Tl::TM, TN = Tl::TN;
  constexpr int A_PER = Tl::A_PER, B_PER = Tl::B_PER;

  __shared__ __attribute__((aligned(16))) bf16_t sA[2][BM][LDK];
  __shared__ __attribute__((aligned(16))) bf16_t sB[2][BN][LDK];

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int wm = wave / WN, wn = wave % WN;
  const int l16 = lane & 15, lg = lane >> 4;

  // ---------------------------------------------------------- tile setup
  int g = 0, row0 = 0, rows = 0, col0 = 0, K = 0;
  if (MODE == GATE_UP) {
    const int i = xcd_tile(*gu.desc_count);
    if (i < 0) return;
    const TileDesc d = gu.desc[i];
    g = d.group; row0 = d.row0; rows = d.rows; col0 = d.col0; K = gu.D;
  } else if (MODE == DOWN) {
    const int i = xcd_tile(*dn.desc_count);
    if (i < 0) return;
    const TileDesc d = dn.desc[i];
    g = d.group; row0 = d.row0; rows = d.rows; col0 = d.col0; K = dn.F;
  } else {
    const int ntiles = cb.D / BN;
    const int mt = blockIdx.x / ntiles, nt = blockIdx.x % ntiles;
    row0 = mt * BM; rows = min(BM, cb.T - row0); col0 = nt * BN; K = cb.Fs;
  }

  // per-thread source pointers of the 16-byte chunks it stages each K step
  const bf16_t* a_src[A_PER];
  const bf16_t* b_src[B_PER];
#pragma unroll
  for (int i = 0; i < A_PER; ++i) {
    const int c = tid + i * NT;
    const int r = min(c / (BK / 8), rows - 1), ch = c % (BK / 8);
    const bf16_t* base;
    if (MODE == GATE_UP) {
      int tok;
      if (g == gu.E) tok = row0 + r;
      else tok = gu.row_assign[gu.offsets[g] + row0 + r] / gu.k;
      base = gu.x + (size_t)tok * gu.D;
    } else if (MODE == DOWN) {
      base = dn.H + (size_t)(dn.offsets[g] + row0 + r) * dn.F;
    } else {
      base = cb.Hs + (size_t)(row0 + r) * cb.Fs;
    }
    a_src[i] = base + ch * 8;
  }
#pragma unroll
  for (int i = 0; i < B_PER; ++i) {
    const int c = tid + i * NT;
    const int n = min(c / (BK / 8), BN - 1), ch = c % (BK / 8);
    const bf16_t* base;
    if (MODE == GATE_UP) {
      const int blk = n / 16, hcol = col0 + (blk / 2) * 16 + (n % 16);
      const bool up = blk & 1;
      if (g == gu.E) base = (up ? gu.sw3 : gu.sw1) + (size_t)hcol * gu.D;
      else base = (up ? gu.w3 : gu.w1) + ((size_t)g * gu.F + hcol) * gu.D;
    } else if (MODE == DOWN) {
      base = dn.w2 + ((size_t)g * dn.D + col0 + n) * dn.F;
    } else {
      base = cb.sw2 + (size_t)(col0 + n) * cb.Fs;
    }
    b_src[i] = base + ch * 8;
  }

  uint4 ra[A_PER], rb[B_PER];
  auto gload = [&](int kt) {
#pragma unroll
    for (int i = 0; i < A_PER; ++i)
      if (Tl::A_CHUNKS % NT == 0 || tid + i * NT < Tl::A_CHUNKS)
        ra[i] = *reinterpret_cast<const uint4*>(a_src[i] + kt * BK);
#pragma unroll
    for (int i = 0; i < B_PER; ++i)
      if (Tl::B_CHUNKS % NT == 0 || tid + i * NT < Tl::B_CHUNKS)
        rb[i] = *reinterpret_cast<const uint4*>(b_src[i] + kt * BK);
  };
  auto lstore = [&](int buf) {
#pragma unroll
    for (int i = 0; i < A_PER; ++i) {
      const int c = tid + i * NT;
      if (Tl::A_CHUNKS % NT == 0 || c < Tl::A_CHUNKS)
        *reinterpret_cast<uint4*>(&sA[buf][c / 8][(c % 8) * 8]) = ra[i];
    }
#pragma unroll
    for (int i = 0; i < B_PER; ++i) {
      const int c = tid + i * NT;
      if (Tl::B_CHUNKS % NT == 0 || c < Tl::B_CHUNKS)
        *reinterpret_cast<uint4*>(&sB[buf][c / 8][(c % 8) * 8]) = rb[i];
    }
  };

  f32x4 acc[FM][FN];
#pragma unroll
  for (int m = 0; m < FM; ++m)
#pragma unroll
    for (int n = 0; n < FN; ++n) acc[m][n] = (f32x4){0.f, 0.f, 0.f, 0.f};

  // 16-row blocks of this wave that hold at least one valid row
  const int live_m = min(FM, max(0, (rows - wm * TM + 15) / 16));

  const int nk = K / BK;
  gload(0);
  lstore(0);
  __syncthreads();
  for (int kt = 0; kt < nk; ++kt) {
    const int cur = kt & 1;
    if (kt + 1 < nk) gload(kt + 1);
#pragma unroll
    for (int s = 0; s < BK / 32; ++s) {
      bf16x8 bfr[FN];
#pragma unroll
      for (int n = 0; n < FN; ++n)
        bfr[n] = *reinterpret_cast<const bf16x8*>(&sB[cur][wn * TN + n * 16 + l16][s * 32 + lg * 8]);
#pragma unroll
      for (int m = 0; m < FM; ++m) {
        if (m < live_m) {
          const bf16x8 afr =
              *reinterpret_cast<const bf16x8*>(&sA[cur][wm * TM + m * 16 + l16][s * 32 + lg * 8]);
#pragma unroll
          for (int n = 0; n < FN; ++n)
            acc[m][n] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(afr, bfr[n], acc[m][n], 0, 0, 0);
        }
      }
    }
    if (kt + 1 < nk) lstore(cur ^ 1);
    __syncthreads();
  }

  // ------------------------------------------------------------ epilogue
  // accumulator element r of block (m, n): row wm*TM + m*16 + 4*lg + r,
  // column wn*TN + n*16 + l16.
  if (MODE == GATE_UP) {
    const bool shared = (g == gu.E);
    const int F = shared ? gu.Fs : gu.F;
    bf16_t* Hb = shared ? gu.Hs + (size_t)row0 * F
                        : gu.H + (size_t)(gu.offsets[g] + row0) * F;
#pragma unroll
    for (int m = 0; m < FM; ++m) {
#pragma unroll
      for (int q = 0; q < FN / 2; ++q) {
        const int hcol = col0 + (wn * TN / 32 + q) * 16 + l16;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int row = wm * TM + m * 16 + 4 * lg + r;
          if (row < rows) {
            const float h = silu(acc[m][2 * q][r]) * acc[m][2 * q + 1][r];
            Hb[(size_t)row * F + hcol] = f32_to_bf16(h);
          }
        }
      }
    }
  } else if (MODE == DOWN) {
    const int prow0 = dn.offsets[g] + row0;
#pragma unroll
    for (int m = 0; m < FM; ++m) {
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int row = wm * TM + m * 16 + 4 * lg + r;
        if (row < rows) {
          const int a = dn.row_assign[prow0 + row];
          const float w = dn.topk_w[a];
          float* y = dn.Y + (size_t)a * dn.D + col0 + wn * TN + l16;
#pragma unroll
          for (int n = 0; n < FN; ++n) y[n * 16] = w * acc[m][n][r];
        }
      }
    }
  } else {
#pragma unroll
    for (int m = 0; m < FM; ++m) {
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int row = wm * TM + m * 16 + 4 * lg + r;
        if (row < rows) {
          const int t = row0 + row;
          const int col = col0 + wn * TN + l16;
          const float* y = cb.Y + (size_t)t * cb.k * cb.D + col;
          float* o = cb.out + (size_t)t * cb.D + col;
#pragma unroll
          for (int n = 0; n < FN; ++n) {
            float v = acc[m][n][r];
            for (int j = 0; j < cb.k; ++j) v += y[(size_t)j * cb.D + n * 16];
            o[n * 16] = v;
          }
        }
      }
    }
  }
}

template <int BM, int BN, int WM, int WN, int MODE>
hipError_t launch_one(const GateUpArgs& gu, const DownArgs& dn, const CombineArgs& cb,
                      unsigned grid, hipStream_t s) {
  grouped_gemm_kernel<BM, BN, WM, WN, MODE><<<grid, WM * WN * kWave, 0, s>>>(gu, dn, cb);
  return hipGetLastError();
}

template <int MODE>
hipError_t dispatch(GemmShape sh, const GateUpArgs& gu, const DownArgs& dn,
                    const CombineArgs& cb, unsigned grid, hipStream_t s) {
  if (sh.BN == 128) {
    if (sh.BM == 16) return launch_one<16, 128, 1, 4, MODE>(gu, dn, cb, grid, s);
    if (sh.BM == 64) return launch_one<64, 128, 1, 4, MODE>(gu, dn, cb, grid, s);
    if (sh.BM == 128) return launch_one<128, 128, 2, 2, MODE>(gu, dn, cb, grid, s);
  }
  if constexpr (MODE != GATE_UP) {
    // output widths that are a multiple of 64 but not of 128
    if (sh.BN == 64) {
      if (sh.BM == 16) return launch_one<16, 64, 1, 2, MODE>(gu, dn, cb, grid, s);
      if (sh.BM == 64) return launch_one<64, 64, 2, 2, MODE>(gu, dn, cb, grid, s);
      if (sh.BM == 128) return launch_one<128, 64, 2, 2, MODE>(gu, dn, cb, grid, s);
    }
  }
  return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_gateup_bf16(const GateUpArgs& a, GemmShape sh, hipStream_t s) {
  return dispatch<GATE_UP>(sh, a, DownArgs{}, CombineArgs{}, (unsigned)a.grid, s);
}

hipError_t launch_down_bf16(const DownArgs& a, GemmShape sh, hipStream_t s) {
  return dispatch<DOWN>(sh, GateUpArgs{}, a, CombineArgs{}, (unsigned)a.grid, s);
}

hipError_t launch_shared_combine_bf16(const CombineArgs& a, GemmShape sh, hipStream_t s) {
  const unsigned grid = (unsigned)(cdiv(a.T, sh.BM) * (a.D / sh.BN));
  return dispatch<SHARED_COMBINE>(sh, GateUpArgs{}, DownArgs{}, a, grid, s);
}

}  // namespace glm
