// Grouped expert GEMMs of the GLM-5.2 MoE layer on gfx950 bf16 MFMA.
//
// Every product here is C[M x N] = A[M x K] . B[N x K]^T with both operands
// K-contiguous: A rows are token activations (gathered through the
// permutation) or gated hidden rows, B rows are weight rows (w1/w3 [F][D],
// w2 [D][F]).  One workgroup computes a BM x BN tile.
//
// Data movement: K is walked in steps of BK through a ring of ST LDS stages,
// each a separate LDS object.  Tiles are copied global -> LDS with gfx950's
// 16-byte LDS-DMA loads (no staging registers), ST-1 steps ahead of the MFMA
// work, and each wave waits only for the oldest stage (vmcnt), so HBM latency
// is covered by up to ST-1 steps of math.  Rows are stored unpadded with the
// 16-byte chunks of each row XOR-swizzled, which keeps the MFMA fragment reads
// free of bank conflicts.  With two stages the copy-first variant (EARLY)
// refills a stage before waiting for the next one.  A tile that is the only
// row tile of its group copies the group's weight rows with the non-temporal
// hint on tiles of up to GLM_STREAM_B_MAX_BM rows (it is their only reader).
//
// Math: each wave owns a (BM/WM) x (BN/WN) sub-tile and accumulates it with
// v_mfma_f32_32x32x16_bf16 (MB = 32) or v_mfma_f32_16x16x32_bf16 (MB = 16).
// The valid rows of a partial tile are split evenly between the wave rows and
// MFMA blocks holding no valid row are skipped.
//
// Epilogues:
//  * GATE_UP: B-tile rows alternate MB rows of w1 (gate) with the matching MB
//    rows of w3 (up), so one lane holds gate and up of the same hidden unit and
//    writes H = bf16(SiLU(g) * u) (SiLU-gated expert MLP with the w1/w3/w2 roles
//    of the PocketLLM "GLM-5.2" page, Implemented execution path).
//  * DOWN: Y[t][j] = w[t][j] * (H W2^T): the routing weight is applied and the
//    row lands in its (token, slot) place (un-permute); no atomics.  The
//    shared expert is group E and writes Y[t][k] with weight 1.  Slot rows are
//    written with non-temporal stores (each is read once, by the combine).
// A streaming kernel then forms out[t] = Y[t][k] + sum_j Y[t][j] in slot
// order: the always-on shared expert merged with the weighted routed outputs
// (GLM-5.2 anatomy page, Mixture of Experts panel).
#include "common.h"

#include <type_traits>

namespace glm {
// Named (not anonymous) so the host launch stubs of the kernel template are
// emitted; the library exports only the C ABI.
namespace gemm {

enum Mode { GATE_UP = 0, DOWN = 1 };

typedef float f32x16 __attribute__((ext_vector_type(16)));

// Physical 16-byte chunk of logical chunk c in row r: c ^ swz(r).  Rows r and
// r+1..r+15 read at one logical chunk land on distinct banks for both 8- and
// 16-lane LDS phases.
template <int BK>
__device__ __forceinline__ int swz(int r) {
  if constexpr (BK == 64) return (r & 7) ^ ((r >> 3) & 1);
  else return ((r >> 1) & 3) ^ ((r >> 3) & 1);
}

template <int BM_, int BN_, int BK_, int WM_, int WN_, int ST_, int MB_>
struct Cfg {
  static constexpr int BM = BM_, BN = BN_, BK = BK_, WM = WM_, WN = WN_, ST = ST_, MB = MB_;
  static constexpr int NW = WM * WN, NT = NW * kWave;
  static constexpr int TM = BM / WM, TN = BN / WN;
  static constexpr int FM = TM / MB, FN = TN / MB;
  static constexpr int CPR = BK / 8;          // 16-byte chunks per row
  static constexpr int RPI = kWave / CPR;     // rows per DMA instruction (1 KB)
  static constexpr int A_INST = BM / RPI, B_INST = BN / RPI;
  static constexpr int IPW = (A_INST + B_INST) / NW;  // DMA instructions per wave per stage
  static constexpr int STAGE = (BM + BN) * BK;        // bf16 elements per stage
  static constexpr int KSUB = BK / (MB == 32 ? 16 : 32);  // MFMA k-steps per stage
  static_assert(TM % MB == 0 && TN % MB == 0, "wave tile must hold whole MFMA blocks");
  static_assert(BM % RPI == 0 && BN % RPI == 0, "tiles must be whole DMA instructions");
  static_assert((A_INST + B_INST) % NW == 0, "every wave issues the same number of DMAs");
  static_assert(A_INST % NW == 0, "copy i of every wave is an A copy exactly when i < A_INST / NW");
  static_assert(BM % 16 == 0 && BN % 16 == 0, "swizzle period");
  static_assert(ST >= 2 && ST <= 8, "ring of 2 to 8 stages");
};

__device__ inline float silu(float g) { return g / (1.0f + expf(-g)); }

// Global address (K offset 0) of row r of a tile's operand rows: r < BM is
// an A row (rows past the tile's valid rows repeat its last valid row), else
// B row r - BM.  Gate/up B rows alternate MB rows of w1 (gate) with the
// matching MB rows of w3 (up).
template <int MODE, int BM, int MB>
__device__ __forceinline__ const bf16_t* tile_row_src(const GateUpArgs& gu, const DownArgs& dn,
                                                      int g, int row0, int rows, int col0, int r) {
  if (r < BM) {
    const int rr = min(r, rows - 1);
    if constexpr (MODE == GATE_UP) {
      const int tok = (g == gu.E) ? row0 + rr : gu.row_assign[row0 + rr] / gu.k;
      return gu.x + (size_t)tok * gu.D;
    } else {
      return (g == dn.E) ? dn.Hs + (size_t)(row0 + rr) * dn.Fs
                         : dn.H + (size_t)(row0 + rr) * dn.F;
    }
  }
  const int n = r - BM;
  if constexpr (MODE == GATE_UP) {
    const int blk = n / MB, hcol = col0 + (blk / 2) * MB + (n % MB);
    const bool up = blk & 1;
    if (g == gu.E) return (up ? gu.sw3 : gu.sw1) + (size_t)hcol * gu.D;
    return (up ? gu.w3 : gu.w1) + ((size_t)g * gu.F + hcol) * gu.D;
  } else {
    return (g == dn.E) ? dn.sw2 + (size_t)(col0 + n) * dn.Fs
                       : dn.w2 + ((size_t)g * dn.D + col0 + n) * dn.F;
  }
}

// Epilogue of a tile: every wave writes its (TM x TN) accumulators.
//  * GATE_UP: H = bf16(SiLU(g) * u) of its hidden columns; with `hblk` (a
//    per-wave LDS scratch of MB x TN/2 bf16, used when GU_LDS) one MB-row block
//    at a time through LDS with 16-byte stores, else straight from the
//    accumulators.
//  * DOWN: Y[t][j] = w * acc to the row's (token, slot) place (the shared
//    group's K chunk kc to slot k + kc); `s_asg` /
//    `s_wt` (BM entries each) take every row's Y row and weight; with `yblk`
//    (a per-wave LDS scratch of MB x TN fp32, used when DN_LDS) through LDS
//    with 16-byte stores.
// The LDS regions may alias the operand stages: the function starts with a
// workgroup barrier after which no wave reads them any more.
template <class C, int MODE, bool GU_LDS, bool DN_LDS, class Acc>
__device__ __forceinline__ void tile_epilogue(const GateUpArgs& gu, const DownArgs& dn,
                                              Acc (&acc)[C::FM][C::FN], int g, int row0, int rows,
                                              int col0, int kc, int wrow0, int live_m, int row_a,
                                              float row_wt, bf16_t* hblk, float* yblk, int* s_asg,
                                              float* s_wt) {
  constexpr int MB = C::MB, FM = C::FM, FN = C::FN, TN = C::TN, WN = C::WN;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, wn = wave % WN;
  const int lr = lane % MB, lk = lane / MB;
  // accumulator element r of block (m, n):
  //   MB = 32: row 8*(r/4) + 4*(lane/32) + r%4, column lane % 32
  //   MB = 16: row 4*(lane/16) + r,             column lane % 16
  constexpr int NR = MB == 32 ? 16 : 4;
  auto row_of = [&](int m, int r) {
    return wrow0 + m * MB + (MB == 32 ? 8 * (r / 4) + 4 * lk + (r % 4) : 4 * lk + r);
  };
  if constexpr (MODE == GATE_UP) {
    const bool shared = (g == gu.E);
    const int F = shared ? gu.Fs : gu.F;
    bf16_t* Hb = (shared ? gu.Hs : gu.H) + (size_t)row0 * F;
    constexpr int HC = TN / 2;  // hidden columns of this wave
    __syncthreads();            // every wave is done reading the stages
    if (kc >= 0) {  // a K chunk: its fp32 sums of gate and up
      float* Pk = gu.P + ((size_t)kc * gu.T + row0) * (2 * gu.pw);
#pragma unroll
      for (int m = 0; m < FM; ++m) {
        if (m >= live_m) continue;
#pragma unroll
        for (int q = 0; q < FN / 2; ++q) {
          const int hcol = col0 + (wn * TN / (2 * MB) + q) * MB + lr - gu.pc0;
#pragma unroll
          for (int r = 0; r < NR; ++r) {
            const int row = row_of(m, r);
            if (row < rows) {
              store_stream(Pk + (size_t)row * (2 * gu.pw) + hcol, acc[m][2 * q][r]);
              store_stream(Pk + (size_t)row * (2 * gu.pw) + gu.pw + hcol, acc[m][2 * q + 1][r]);
            }
          }
        }
      }
      return;
    }
    if constexpr (GU_LDS) {
      // Through LDS, one MB-row block at a time (as the down epilogue):
      // 16-byte stores of 8 consecutive hidden values.
      constexpr int CG = HC / 8 > 0 ? HC / 8 : 1, RPP = kWave / CG;
      static_assert(kWave % CG == 0 && MB % RPP == 0, "epilogue pass shape");
      const int hcol0 = col0 + wn * HC;
#pragma unroll
      for (int m = 0; m < FM; ++m) {
        if (m >= live_m) continue;
#pragma unroll
        for (int q = 0; q < FN / 2; ++q)
#pragma unroll
          for (int r = 0; r < NR; ++r) {
            const int rb = row_of(m, r) - (wrow0 + m * MB);
            const float h = silu(acc[m][2 * q][r]) * acc[m][2 * q + 1][r];
            hblk[rb * HC + q * MB + lr] = f32_to_bf16(h);
          }
#pragma unroll
        for (int pass = 0; pass < MB / RPP; ++pass) {
          const int rb = pass * RPP + lane / CG, cg = lane % CG;
          const int row = wrow0 + m * MB + rb;
          const uint4 v = *reinterpret_cast<const uint4*>(hblk + rb * HC + 8 * cg);
          if (row < rows) *reinterpret_cast<uint4*>(Hb + (size_t)row * F + hcol0 + 8 * cg) = v;
        }
      }
    } else {
#pragma unroll
      for (int m = 0; m < FM; ++m) {
        if (m >= live_m) continue;
#pragma unroll
        for (int q = 0; q < FN / 2; ++q) {
          const int hcol = col0 + (wn * TN / (2 * MB) + q) * MB + lr;
#pragma unroll
          for (int r = 0; r < NR; ++r) {
            const int row = row_of(m, r);
            if (row < rows) {
              const float h = silu(acc[m][2 * q][r]) * acc[m][2 * q + 1][r];
              Hb[(size_t)row * F + hcol] = f32_to_bf16(h);
            }
          }
        }
      }
    }
  } else {
    __syncthreads();  // every wave is done reading the stages (s_asg may alias one)
    // row of Y and routing weight of every row of the tile
    if (tid < rows) {  // the shared group's K chunk kc writes slot k + kc
      s_asg[tid] = g == dn.E ? (row0 + tid) * (dn.k + dn.ksplit) + dn.k + kc
                             : y_row(row_a, dn.k);
      s_wt[tid] = row_wt;
    }
    __syncthreads();  // the row table is complete
    if constexpr (DN_LDS) {
      // Through LDS, one MB-row block at a time: each wave writes its block
      // (MB x TN fp32) to its own scratch, then stores whole 16-byte column
      // groups, so a store instruction covers a few full row pieces.
      constexpr int CG = TN / 4;            // 16-byte column groups per row
      constexpr int RPP = kWave / CG;       // rows per pass
      static_assert(kWave % CG == 0 && MB % RPP == 0, "epilogue pass shape");
#pragma unroll
      for (int m = 0; m < FM; ++m) {
        if (m >= live_m) continue;
#pragma unroll
        for (int r = 0; r < NR; ++r) {
          const int rb = row_of(m, r) - (wrow0 + m * MB);
#pragma unroll
          for (int n = 0; n < FN; ++n) yblk[rb * TN + n * MB + lr] = acc[m][n][r];
        }
#pragma unroll
        for (int pass = 0; pass < MB / RPP; ++pass) {
          const int rb = pass * RPP + lane / CG, cg = lane % CG;
          const int row = wrow0 + m * MB + rb;
          const float4 v = *reinterpret_cast<const float4*>(yblk + rb * TN + 4 * cg);
          if (row < rows) {
            const float w = s_wt[row];
            float* y = dn.Y + (size_t)s_asg[row] * dn.D + col0 + wn * TN + 4 * cg;
            store_stream(y, f32x4{w * v.x, w * v.y, w * v.z, w * v.w});
          }
        }
      }
    } else {
#pragma unroll
      for (int m = 0; m < FM; ++m) {
        if (m >= live_m) continue;
#pragma unroll
        for (int r = 0; r < NR; ++r) {
          const int row = row_of(m, r);
          if (row < rows) {
            const float w = s_wt[row];
            float* y = dn.Y + (size_t)s_asg[row] * dn.D + col0 + wn * TN + lr;
#pragma unroll
            for (int n = 0; n < FN; ++n) store_stream(y + n * MB, w * acc[m][n][r]);
          }
        }
      }
    }
  }
}



// EARLY (two stages only): each stage's refill is issued before the wait for
// the next stage instead of after it (see the main loop).
#ifndef GLM_LIVE_A  // uniform-ring kernel: copy only the live row blocks' A rows
#define GLM_LIVE_A 1
#endif
template <class C, int MODE, bool EARLY>
__global__ __launch_bounds__(C::NT) void grouped_gemm_kernel(GateUpArgs gu, DownArgs dn) {
  constexpr int BM = C::BM, BN = C::BN, BK = C::BK, ST = C::ST, MB = C::MB;
  constexpr int WN = C::WN, NW = C::NW, TM = C::TM, TN = C::TN, FM = C::FM, FN = C::FN;
  constexpr int CPR = C::CPR, RPI = C::RPI, IPW = C::IPW;

  __shared__ __attribute__((aligned(1024))) bf16_t lds0[C::STAGE];
  __shared__ __attribute__((aligned(1024))) bf16_t lds1[C::STAGE];
  __shared__ __attribute__((aligned(1024))) bf16_t lds2[ST > 2 ? C::STAGE : 8];
  __shared__ __attribute__((aligned(1024))) bf16_t lds3[ST > 3 ? C::STAGE : 8];
  __shared__ __attribute__((aligned(1024))) bf16_t lds4[ST > 4 ? C::STAGE : 8];
  __shared__ __attribute__((aligned(1024))) bf16_t lds5[ST > 5 ? C::STAGE : 8];
  __shared__ __attribute__((aligned(1024))) bf16_t lds6[ST > 6 ? C::STAGE : 8];
  __shared__ __attribute__((aligned(1024))) bf16_t lds7[ST > 7 ? C::STAGE : 8];
  __shared__ int s_asg[BM];
  __shared__ float s_wt[BM];

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int wm = wave / WN, wn = wave % WN;

  // ---------------------------------------------------------- tile setup
  int g = 0, row0 = 0, rows = 0, col0 = 0, K = 0, kc = 0, koff = 0;
  bool sole = false;
  if constexpr (MODE == GATE_UP) {
    const int i = xcd_tile(*gu.desc_count, gu.xblk);
    if (i < 0) return;
    const TileDesc d = gu.desc[i];
    g = d.group & kGroupMask; sole = d.group & kSoleRowTile; row0 = d.row0; rows = d.rows;
    col0 = d.col0; K = gu.D;
    kc = -1;
    if (d.group & kChunkTile) {  // one K chunk of a shared-group tile
      kc = d.group >> kKChunkShift;
      K = gu.D / gu.ksplit;
      koff = kc * K;
    }
  } else {
    const int i = xcd_tile(*dn.desc_count, dn.xblk);
    if (i < 0) return;
    const TileDesc d = dn.desc[i];
    g = d.group & kGroupMask; sole = d.group & kSoleRowTile; row0 = d.row0; rows = d.rows;
    col0 = d.col0;
    K = dn.F;
    if (g == dn.E) {  // the shared group, possibly one K chunk of it
      kc = d.group >> kKChunkShift;
      K = dn.Fs / dn.ksplit;
      koff = kc * K;
    }
  }

  // MFMA row blocks holding valid rows, dealt to the wave rows in turn as
  // evenly as possible: a SIMD runs one wave of each wave row, so its MFMA
  // work is the blocks of both (ceil(rows / MB) in all, not WM x the larger)
  const int nb = (rows + MB - 1) / MB;
  const int live_m = min(FM, nb / C::WM + (wm < nb % C::WM ? 1 : 0));
  const int wrow0 = MB * (wm * (nb / C::WM) + min(wm, nb % C::WM));

  // DMA sources: instruction q = wave + i*NW covers rows [q*RPI, q*RPI+RPI) of
  // the stage (A rows first, then B rows); lane l fills physical chunk l % CPR
  // of row q*RPI + l / CPR, i.e. logical chunk (l % CPR) ^ swz(row).
  const bf16_t* src[IPW];
#pragma unroll
  for (int i = 0; i < IPW; ++i) {
    const int q = wave + i * NW;
    const int r = q * RPI + lane / CPR;
    const int ch = (lane % CPR) ^ swz<BK>(r);
    src[i] = tile_row_src<MODE, BM, MB>(gu, dn, g, row0, rows, col0, r) + koff + ch * 8;
  }
  // LIVEA (the waves of a wave row cover one row block per copy): instead,
  // wave (wm, wn) copies rows wn*RPI .. +RPI of each live row block of its
  // wave row, LIVE A copies a stage, so rows of blocks past the valid rows
  // are never fetched (their LDS rows reach no MFMA), and BW weight-row
  // copies: B copy i covers B rows (wave + i*NW)*RPI .. +RPI.
  constexpr bool LIVEA = GLM_LIVE_A && C::WN * RPI == MB && C::B_INST % NW == 0;
  constexpr int BW = C::B_INST / NW;
  const bf16_t* sa_l[LIVEA ? FM : 1];
  int a_dst[LIVEA ? FM : 1];
  const bf16_t* sb_l[LIVEA ? BW : 1];
  if constexpr (LIVEA) {
#pragma unroll
    for (int i = 0; i < FM; ++i) {
      a_dst[i] = min(wrow0 + i * MB, BM - MB) + wn * RPI;
      const int r = a_dst[i] + lane / CPR;
      sa_l[i] = tile_row_src<MODE, BM, MB>(gu, dn, g, row0, rows, col0, r) + koff +
                ((lane % CPR) ^ swz<BK>(r)) * 8;
    }
#pragma unroll
    for (int i = 0; i < BW; ++i) {
      const int r = BM + (wave + i * NW) * RPI + lane / CPR;
      sb_l[i] = tile_row_src<MODE, BM, MB>(gu, dn, g, row0, rows, col0, r) + koff +
                ((lane % CPR) ^ swz<BK>(r)) * 8;
    }
  }

  // Per-row data of the down epilogue (assignment and routing weight of row
  // `tid` of the tile): loaded into registers before the first copies are
  // issued and written to LDS only at the epilogue, so the loads' latency
  // stays off the path to the first K step.
  static_assert(BM <= C::NT, "one epilogue row per thread");
  int row_a = 0;
  float row_wt = 1.0f;
  if constexpr (MODE == DOWN) {
    if (tid < rows && g != dn.E) {
      row_a = dn.row_assign[row0 + tid];
      row_wt = dn.row_w[row0 + tid];
    }
  }

  auto stage_ptr = [&](int s) -> bf16_t* {
    return s == 0 ? lds0 : s == 1 ? lds1 : s == 2 ? lds2 : s == 3 ? lds3
         : s == 4 ? lds4 : s == 5 ? lds5 : s == 6 ? lds6 : lds7;
  };
  // NT: weight rows go with the non-temporal hint (a sole row tile, see kStreamB)
  auto issue = [&](bf16_t* st, int kt, auto nt_c) {
    constexpr bool NT = decltype(nt_c)::value;
#pragma unroll
    for (int i = 0; i < IPW; ++i) {
      const int q = wave + i * NW;
      // (the source goes through void*: a typed pointer here silently drops
      // the kernel's host-side launch stub)
      if (NT && i * NW >= C::A_INST)  // a weight-row copy
        __builtin_amdgcn_global_load_lds((const void*)(src[i] + (size_t)kt * BK),
                                         (lds_void*)(st + q * (RPI * BK)), 16, 0, kCpolNt);
      else
        __builtin_amdgcn_global_load_lds((const void*)(src[i] + (size_t)kt * BK),
                                         (lds_void*)(st + q * (RPI * BK)), 16, 0, 0);
    }
  };

  // copies of step kt into stage st: LIVE A copies and BW B copies (LIVEA),
  // else the IPW uniform copies
  auto issue_any = [&](bf16_t* st, int kt, auto nt_c, auto live_c) {
    if constexpr (LIVEA) {
      constexpr bool NT = decltype(nt_c)::value;
      constexpr int LIVE = decltype(live_c)::value;
#pragma unroll
      for (int i = 0; i < LIVE; ++i)
        __builtin_amdgcn_global_load_lds((const void*)(sa_l[i] + (size_t)kt * BK),
                                         (lds_void*)(st + a_dst[i] * BK), 16, 0, 0);
#pragma unroll
      for (int i = 0; i < BW; ++i)
        __builtin_amdgcn_global_load_lds((const void*)(sb_l[i] + (size_t)kt * BK),
                                         (lds_void*)(st + (BM + (wave + i * NW) * RPI) * BK),
                                         16, 0, NT ? kCpolNt : 0);
    } else {
      issue(st, kt, nt_c);
    }
  };

  // fragment read offsets (elements, without the stage base and k-chunk)
  const int lr = lane % MB, lk = lane / MB;
  const int sw = swz<BK>(lr);

  typedef typename std::conditional<MB == 32, f32x16, f32x4>::type acc_t;
  acc_t acc[FM][FN];
#pragma unroll
  for (int m = 0; m < FM; ++m)
#pragma unroll
    for (int n = 0; n < FN; ++n) acc[m][n] = acc_t{};

  const int nk = K / BK;
  constexpr bool early = EARLY && ST == 2;
  static_assert(!EARLY || ST == 2, "copy-before-wait order needs two stages");

  // Main loop, specialised on the number of live MFMA row blocks (LIVE) so the
  // inner loop has no branches.  Software pipeline per stage: reads of
  // sub-step s+1 are issued before the MFMAs of sub-step s, and the stage
  // hand-over (wait, barrier, refill, next stage's first reads) sits just
  // before the last sub-step's MFMAs.
  auto run = [&](auto live_c, auto nt_c) {
    constexpr int LIVE = decltype(live_c)::value;
    constexpr int VPS = LIVEA ? LIVE + BW : IPW;  // this wave's copies per stage
    bf16x8 fa[2][FM], fb[2][FN];
    auto load_frags = [&](const bf16_t* st, int sub, int slot) {
      const int kc = (MB == 32 ? 2 * sub : 4 * sub) + lk;  // logical 16-byte chunk
      const int off = (kc ^ sw) * 8;
      const bf16_t* sa = st + (wrow0 + lr) * BK + off;
      const bf16_t* sb = st + (BM + wn * TN + lr) * BK + off;
#pragma unroll
      for (int n = 0; n < FN; ++n)
        fb[slot][n] = *reinterpret_cast<const bf16x8*>(sb + n * MB * BK);
#pragma unroll
      for (int m = 0; m < LIVE; ++m)
        fa[slot][m] = *reinterpret_cast<const bf16x8*>(sa + m * MB * BK);
    };
    auto mma = [&](int slot) {
#pragma unroll
      for (int m = 0; m < LIVE; ++m)
#pragma unroll
        for (int n = 0; n < FN; ++n) {
          if constexpr (MB == 32)
            acc[m][n] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[slot][m], fb[slot][n],
                                                                acc[m][n], 0, 0, 0);
          else
            acc[m][n] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fa[slot][m], fb[slot][n],
                                                                acc[m][n], 0, 0, 0);
        }
    };
    // prologue: fill every stage, wait for stage 0, read its first fragments
#pragma unroll
    for (int s = 0; s < ST; ++s)
      if (s < nk) issue_any(stage_ptr(s), s, nt_c, live_c);
    if (ST - 1 < nk) __builtin_amdgcn_s_waitcnt(GLM_VMCNT(VPS * (ST - 1)));
    else __builtin_amdgcn_s_waitcnt(GLM_VMCNT(0));
    lds_barrier();
    load_frags(stage_ptr(0), 0, 0);

    auto step = [&](auto sc, int kt) {
      constexpr int s = decltype(sc)::value;  // stage of k-step kt
      bf16_t* cur = stage_ptr(s);
#pragma unroll
      for (int sub = 0; sub < C::KSUB; ++sub) {
        if (sub + 1 < C::KSUB) load_frags(cur, sub + 1, (sub + 1) & 1);
        if (sub == C::KSUB - 1 && kt + 1 < nk) {
          // Every read of this stage is issued (the last sub-step's fragments
          // are in registers), so before its MFMAs: wait for stage kt+1 (stages
          // kt+2 .. kt+ST-1 may stay in flight), meet the barrier, refill this
          // stage ST steps ahead and read the next stage's first fragments;
          // the MFMAs below then cover that read latency.
          if constexpr (early) {
            // The refill of this stage goes out before the wait for the next
            // one, so a copy is always in flight; a second barrier then tells
            // every wave that all copies of stage kt+1 have landed.
            lds_barrier();  // every wave is done reading stage kt
            if (kt + 2 < nk) {
              issue_any(cur, kt + 2, nt_c, live_c);
              __builtin_amdgcn_s_waitcnt(GLM_VMCNT(VPS));  // this wave's copies of kt+1
            } else {
              __builtin_amdgcn_s_waitcnt(GLM_VMCNT(0));
            }
            asm volatile("s_barrier" ::: "memory");
          } else {
            if (kt + ST - 1 < nk) __builtin_amdgcn_s_waitcnt(GLM_VMCNT(VPS * (ST - 2)));
            else __builtin_amdgcn_s_waitcnt(GLM_VMCNT(0));
            lds_barrier();
            if (kt + ST < nk) issue_any(cur, kt + ST, nt_c, live_c);
          }
          load_frags(stage_ptr((s + 1) % ST), 0, 0);  // slot 0 is free: sub-step KSUB-2 used it
        }
        // Pin the reads issued above ahead of this sub-step's MFMAs: left free,
        // the scheduler sinks each read to its first MFMA and waits at once.
        __builtin_amdgcn_sched_barrier(0);
        mma(sub & 1);
      }
    };
    for (int kt = 0; kt < nk; kt += ST) {
      unroll<ST>([&](auto uc) {
        constexpr int u = decltype(uc)::value;
        if (u == 0 || kt + u < nk) step(std::integral_constant<int, u>{}, kt + u);
      });
    }
  };
  static_assert(C::KSUB % 2 == 0, "fragment slots alternate per sub-step");
  static_assert(FM <= 4, "live-block dispatch covers up to 4 row blocks");
  // the main loop, specialised on the live row blocks and the copy hint
  auto go = [&](auto nt_c) {
    switch (live_m) {
      case 1: run(std::integral_constant<int, 1>{}, nt_c); break;
      case 2: if constexpr (FM >= 2) run(std::integral_constant<int, 2>{}, nt_c); break;
      case 3: if constexpr (FM >= 3) run(std::integral_constant<int, 3>{}, nt_c); break;
      case 4: if constexpr (FM >= 4) run(std::integral_constant<int, 4>{}, nt_c); break;
      default: {
        // this wave row holds no valid row: make its copies (LIVEA: weight
        // rows only) and keep the barrier count of the others
        const std::integral_constant<int, 0> none{};
        constexpr int VPS0 = LIVEA ? BW : IPW;
        for (int s = 0; s < ST; ++s)
          if (s < nk) issue_any(stage_ptr(s), s, nt_c, none);
        __builtin_amdgcn_s_waitcnt(GLM_VMCNT(0));
        lds_barrier();
        for (int kt = 0; kt + 1 < nk; ++kt) {
          if constexpr (early) {  // the same two barriers per step as the other waves
            lds_barrier();
            if (kt + 2 < nk) {
              issue_any(stage_ptr(kt % ST), kt + 2, nt_c, none);
              __builtin_amdgcn_s_waitcnt(GLM_VMCNT(VPS0));
            } else {
              __builtin_amdgcn_s_waitcnt(GLM_VMCNT(0));
            }
            asm volatile("s_barrier" ::: "memory");
          } else {
            __builtin_amdgcn_s_waitcnt(GLM_VMCNT(0));
            lds_barrier();
            if (kt + ST < nk) issue_any(stage_ptr(kt % ST), kt + ST, nt_c, none);
          }
        }
      }
    }
  };
  if constexpr (kStreamB<BM, BN>) {
    if (sole) go(std::true_type{});
    else go(std::false_type{});
  } else {
    go(std::false_type{});
  }

  // ------------------------------------------------------------ epilogue
  // (through LDS where stage 0 is large enough for every wave's block)
  constexpr int HC = TN / 2;
  constexpr bool GU_LDS = NW * MB * HC * 2 <= C::STAGE * 2 && HC % 8 == 0 &&
                          MB % (kWave / (HC / 8 > 0 ? HC / 8 : 1)) == 0;
  constexpr bool DN_LDS = NW * MB * TN * 4 <= C::STAGE * 2;
  tile_epilogue<C, MODE, GU_LDS, DN_LDS>(gu, dn, acc, g, row0, rows, col0, kc, wrow0, live_m,
                                         row_a, row_wt,
                         GU_LDS ? lds0 + wave * (MB * HC) : nullptr,
                         DN_LDS ? reinterpret_cast<float*>(lds0) + wave * (MB * TN) : nullptr,
                         s_asg, s_wt);
}

#ifndef GLM_SPREAD_B  // spread the weight copies over the sub-steps (split rings)
#define GLM_SPREAD_B 1
#endif
#ifndef GLM_SPREAD_PARTS  // ... over this many of them, the first ones
#define GLM_SPREAD_PARTS 4
#endif
#ifndef GLM_SPREAD_MID  // ... each after its sub-step's first row block of MFMAs
#define GLM_SPREAD_MID 1
#endif
// Split rings for the 256 x 256 prefill tiles.  The A rows (token
// activations or hidden rows: each is re-read by every column tile of its
// group, so mostly L2 hits) and the B rows (weights: streamed from HBM by the
// first tile that needs them) go through separate rings of 32 KB slots: two
// A slots and three B slots (the whole 160 KB of LDS).  At the end of step kt
// a wave waits for step kt+1, meets the workgroup barrier and refills the
// slots step kt used with the A rows of step kt+2 and the B rows of step
// kt+3, so the weight rows run two K steps ahead of the math with one
// barrier per step.  (With GLM_SPREAD_B the B rows of step kt+2 are issued
// during step kt instead, one copy per sub-step after that sub-step's first
// row block of MFMAs, into the slot step kt-1 left.)  Each slot is its own
// LDS object, so the compiler tracks the LDS-DMA copies per slot.  Rows are
// 128-byte pieces (K step 64): a narrower step would issue two requests per
// cache line.
template <class C, int MODE, int NA, int NB>
__global__ __launch_bounds__(C::NT) void split_gemm_kernel(GateUpArgs gu, DownArgs dn) {
  constexpr int BM = C::BM, BN = C::BN, BK = C::BK, MB = C::MB;
  constexpr int WN = C::WN, NW = C::NW, TM = C::TM, TN = C::TN, FM = C::FM, FN = C::FN;
  constexpr int CPR = C::CPR, RPI = C::RPI;
  constexpr int AW = C::A_INST / NW, BW = C::B_INST / NW;  // copies per wave and step
  static_assert(C::A_INST % NW == 0 && C::B_INST % NW == 0, "whole copies per wave");
  static_assert(C::KSUB % 2 == 0 && FM <= 4, "fragment slots and live-block dispatch");
  constexpr int HC = TN / 2;
  static_assert(NW * MB * HC <= BM * BK && (NW / 2) * MB * TN * 2 <= BN * BK &&
                    2 * BM * 4 <= BM * BK * 2,
                "epilogue scratch fits the ring slots");

  static_assert(BM == BN && NA + NB == 5 && NA >= 2 && NB >= 2 && NA != NB,
                "five equal slots: the A ring takes NA, the B ring NB");
  __shared__ __attribute__((aligned(1024))) bf16_t ls0[BM * BK];
  __shared__ __attribute__((aligned(1024))) bf16_t ls1[BM * BK];
  __shared__ __attribute__((aligned(1024))) bf16_t ls2[BM * BK];
  __shared__ __attribute__((aligned(1024))) bf16_t ls3[BM * BK];
  __shared__ __attribute__((aligned(1024))) bf16_t ls4[BM * BK];

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int wm = wave / WN, wn = wave % WN;

  int g = 0, row0 = 0, rows = 0, col0 = 0, K = 0, kc = 0, koff = 0;
  if constexpr (MODE == GATE_UP) {
    const int i = xcd_tile(*gu.desc_count, gu.xblk);
    if (i < 0) return;
    const TileDesc d = gu.desc[i];
    g = d.group & kGroupMask; row0 = d.row0; rows = d.rows; col0 = d.col0; K = gu.D;
    kc = -1;
    if (d.group & kChunkTile) {  // one K chunk of a shared-group tile
      kc = d.group >> kKChunkShift;
      K = gu.D / gu.ksplit;
      koff = kc * K;
    }
  } else {
    const int i = xcd_tile(*dn.desc_count, dn.xblk);
    if (i < 0) return;
    const TileDesc d = dn.desc[i];
    g = d.group & kGroupMask; row0 = d.row0; rows = d.rows; col0 = d.col0;
    K = dn.F;
    if (g == dn.E) {  // the shared group, possibly one K chunk of it
      kc = d.group >> kKChunkShift;
      K = dn.Fs / dn.ksplit;
      koff = kc * K;
    }
  }

  // MFMA row blocks dealt to the wave rows as evenly as possible: a SIMD
  // runs one wave of each wave row, so its MFMA work is the blocks of both
  const int nb = (rows + MB - 1) / MB;
  const int live_m = min(FM, nb / C::WM + (wm < nb % C::WM ? 1 : 0));
  const int wrow0 = MB * (wm * (nb / C::WM) + min(wm, nb % C::WM));

  // A copies: copy c of wave (wm, wn) fills rows (c*WN + wn)*RPI .. +RPI of
  // each MFMA row block of its wave row, so it makes exactly CPB A copies per
  // live block and rows of blocks past the valid rows are never fetched (the
  // LDS rows they would fill reach only output rows that the epilogue drops).
  // B copy i of a wave covers rows (wave + i*NW)*RPI .. +RPI.  Lane l fills
  // physical chunk l % CPR of its row, logical chunk (l % CPR) ^ swz.
  constexpr int CPB = MB / (WN * RPI);  // A copies per live block per wave
  static_assert(CPB >= 1 && CPB * WN * RPI == MB, "a wave row's copies cover whole row blocks");
  const bf16_t* sa[FM * CPB];
  int a_dst[FM * CPB];
#pragma unroll
  for (int i = 0; i < FM * CPB; ++i) {
    a_dst[i] = min(wrow0 + (i / CPB) * MB, BM - MB) + ((i % CPB) * WN + wn) * RPI;
    const int r = a_dst[i] + lane / CPR;
    sa[i] = tile_row_src<MODE, BM, MB>(gu, dn, g, row0, rows, col0, r) + koff +
            ((lane % CPR) ^ swz<BK>(r)) * 8;
  }
  const bf16_t* sb[BW];
#pragma unroll
  for (int i = 0; i < BW; ++i) {
    const int n = (wave + i * NW) * RPI + lane / CPR;
    sb[i] = tile_row_src<MODE, BM, MB>(gu, dn, g, row0, rows, col0, BM + n) + koff +
            ((lane % CPR) ^ swz<BK>(n)) * 8;
  }

  static_assert(BM <= C::NT, "one epilogue row per thread");
  int row_a = 0;
  float row_wt = 1.0f;
  if constexpr (MODE == DOWN) {
    if (tid < rows && g != dn.E) {
      row_a = dn.row_assign[row0 + tid];
      row_wt = dn.row_w[row0 + tid];
    }
  }

  auto slot = [&](int i) -> bf16_t* {
    return i == 0 ? ls0 : i == 1 ? ls1 : i == 2 ? ls2 : i == 3 ? ls3 : ls4;
  };
  auto a_slot = [&](int s) -> bf16_t* { return slot(s); };
  auto b_slot = [&](int s) -> bf16_t* { return slot(NA + s); };
  // LIVE: the wave row's live blocks (compile time); the wave makes LIVE * CPB A copies a step
  auto issueA = [&](auto live_c, bf16_t* st, int kt) {
    constexpr int LIVE = decltype(live_c)::value;
#pragma unroll
    for (int i = 0; i < LIVE * CPB; ++i)
      __builtin_amdgcn_global_load_lds((const void*)(sa[i] + (size_t)kt * BK),
                                       (lds_void*)(st + a_dst[i] * BK), 16, 0, 0);
  };
  auto issueB = [&](bf16_t* st, int kt) {
#pragma unroll
    for (int i = 0; i < BW; ++i)
      __builtin_amdgcn_global_load_lds((const void*)(sb[i] + (size_t)kt * BK),
                                       (lds_void*)(st + (wave + i * NW) * (RPI * BK)), 16, 0, 0);
  };
  // SPREAD: the B copies of step kt+NB-1 are issued during step kt, BW/KSUB
  // per sub-step, instead of all at the hand-over: a wave then never stalls
  // on a burst of copies while its MFMAs wait to issue.
  constexpr int PARTS = GLM_SPREAD_PARTS < C::KSUB ? GLM_SPREAD_PARTS : C::KSUB;
  constexpr bool SPREAD = GLM_SPREAD_B && NA < NB && BW % PARTS == 0;
  auto issueB_part = [&](bf16_t* st, int kt, int part) {
    constexpr int BPS = BW / PARTS;
    if (part >= PARTS) return;
#pragma unroll
    for (int j = 0; j < BPS; ++j) {
      const int i = part * BPS + j;
      __builtin_amdgcn_global_load_lds((const void*)(sb[i] + (size_t)kt * BK),
                                       (lds_void*)(st + (wave + i * NW) * (RPI * BK)), 16, 0, 0);
    }
  };

  const int nk = K / BK;
  // The shallower ring's copies of a step are issued before the deeper
  // ring's: then at the end of step kt the only copies issued after step
  // kt+1's are the deeper ring's copies of step kt+2.
  constexpr bool A_FIRST = NA < NB;
  constexpr int NMAX = NA > NB ? NA : NB;
  auto issue_step = [&](auto live_c, int st) {  // the copies of step st in the prologue
    if (A_FIRST) {
      if (st < NA) issueA(live_c, a_slot(st), st);
      if (st < (SPREAD ? NB - 1 : NB)) issueB(b_slot(st), st);  // (SPREAD: step 0 copies B of NB-1)
    } else {
      if (st < NB) issueB(b_slot(st), st);
      if (st < NA) issueA(live_c, a_slot(st), st);
    }
  };
  // Steps 0 .. NMAX-1 in step order; wait for step 0
  auto prologue = [&](auto live_c) {
    constexpr int AWL = decltype(live_c)::value * CPB;  // A copies per step
    issue_step(live_c, 0);
    if (nk > 1) issue_step(live_c, 1);
    if (nk > 2) {
      issue_step(live_c, 2);
      __builtin_amdgcn_s_waitcnt(
          GLM_VMCNT(AWL + BW + (NA > 2 ? AWL : 0) + (NB > 2 && !SPREAD ? BW : 0)));
    } else {
      __builtin_amdgcn_s_waitcnt(GLM_VMCNT(0));
    }
    lds_barrier();
  };
  // End of step kt: wait for step kt+1 (the deeper ring's copies of step
  // kt+2 may stay in flight), barrier, refill the slots step kt used.
  // STEADY: steps kt+1 .. kt+NMAX exist (known at compile time).
  auto handover = [&](auto live_c, auto sc, int kt, auto steady_c) {
    constexpr int u = decltype(sc)::value;  // kt % 6
    constexpr bool STEADY = decltype(steady_c)::value;
    constexpr int DEEP_W = A_FIRST ? BW : decltype(live_c)::value * CPB;
    if (STEADY || kt + 2 < nk) __builtin_amdgcn_s_waitcnt(GLM_VMCNT(DEEP_W));
    else __builtin_amdgcn_s_waitcnt(GLM_VMCNT(0));
    lds_barrier();
    if (A_FIRST) {
      if (STEADY || kt + NA < nk) issueA(live_c, a_slot(u % NA), kt + NA);
      if (!SPREAD && (STEADY || kt + NB < nk)) issueB(b_slot(u % NB), kt + NB);
    } else {
      if (STEADY || kt + NB < nk) issueB(b_slot(u % NB), kt + NB);
      if (STEADY || kt + NA < nk) issueA(live_c, a_slot(u % NA), kt + NA);
    }
  };

  const int lr = lane % MB, lk = lane / MB;
  const int sw = swz<BK>(lr);

  typedef f32x16 acc_t;
  static_assert(MB == 32, "32 x 32 MFMA blocks");
  acc_t acc[FM][FN];
#pragma unroll
  for (int m = 0; m < FM; ++m)
#pragma unroll
    for (int n = 0; n < FN; ++n) acc[m][n] = acc_t{};

  auto run = [&](auto live_c) {
    constexpr int LIVE = decltype(live_c)::value;
    bf16x8 fa[2][FM], fb[2][FN];
    auto load_frags = [&](const bf16_t* sa_, const bf16_t* sb_, int sub, int slot) {
      const int off = ((2 * sub + lk) ^ sw) * 8;
      const bf16_t* pa = sa_ + (wrow0 + lr) * BK + off;
      const bf16_t* pb = sb_ + (wn * TN + lr) * BK + off;
#pragma unroll
      for (int n = 0; n < FN; ++n)
        fb[slot][n] = *reinterpret_cast<const bf16x8*>(pb + n * MB * BK);
#pragma unroll
      for (int m = 0; m < LIVE; ++m)
        fa[slot][m] = *reinterpret_cast<const bf16x8*>(pa + m * MB * BK);
    };
    // MFMAs of row blocks [m0, m1) of a sub-step
    auto mma_rows = [&](int slot, int m0, int m1) {
#pragma unroll
      for (int m = 0; m < LIVE; ++m)
#pragma unroll
        for (int n = 0; n < FN; ++n)
          if (m >= m0 && m < m1)
            acc[m][n] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[slot][m], fb[slot][n],
                                                                acc[m][n], 0, 0, 0);
    };
    auto mma = [&](int slot) { mma_rows(slot, 0, LIVE); };
    prologue(live_c);
    load_frags(a_slot(0), b_slot(0), 0, 0);
    // one K step on the slots of step kt (u = kt % 6); the hand-over sits
    // before the last sub-step's MFMAs, which cover the next slots' first reads
    auto step = [&](auto sc, int kt, auto steady_c) {
      constexpr int u = decltype(sc)::value;
      constexpr bool STEADY = decltype(steady_c)::value;
      const bf16_t* ca = a_slot(u % NA);
      const bf16_t* cb = b_slot(u % NB);
#pragma unroll
      for (int sub = 0; sub < C::KSUB; ++sub) {
        if (sub + 1 < C::KSUB) load_frags(ca, cb, sub + 1, (sub + 1) & 1);
        // (the last sub-step's part before the hand-over: its wait counts
        // these as the youngest copies; the others after the first row
        // block's MFMAs, so the MFMA pipe is busy while the copies issue)
        const bool part = SPREAD && (STEADY || kt + NB - 1 < nk);
        const bool mid = GLM_SPREAD_MID && sub + 1 < C::KSUB && LIVE > 1;
        if (part && !mid) issueB_part(b_slot((u + NB - 1) % NB), kt + NB - 1, sub);
        if (sub == C::KSUB - 1 && (STEADY || kt + 1 < nk)) {
          handover(live_c, sc, kt, steady_c);
          load_frags(a_slot((u + 1) % NA), b_slot((u + 1) % NB), 0, 0);
        }
        // keep the reads issued above ahead of this sub-step's MFMAs
        __builtin_amdgcn_sched_barrier(0);
        if (mid) {
          mma_rows(sub & 1, 0, 1);
          __builtin_amdgcn_sched_barrier(0);
          if (part) issueB_part(b_slot((u + NB - 1) % NB), kt + NB - 1, sub);
          __builtin_amdgcn_sched_barrier(0);
          mma_rows(sub & 1, 1, LIVE);
        } else {
          mma(sub & 1);
        }
      }
    };
    int kt = 0;
    for (; kt + 5 + NMAX < nk; kt += 6)  // every step of the group has NMAX steps after it
      unroll<6>([&](auto uc) { step(uc, kt + decltype(uc)::value, std::true_type{}); });
    for (; kt < nk; kt += 6)
      unroll<6>([&](auto uc) {
        if (kt + decltype(uc)::value < nk) step(uc, kt + decltype(uc)::value, std::false_type{});
      });
  };
  switch (live_m) {
    case 1: run(std::integral_constant<int, 1>{}); break;
    case 2: run(std::integral_constant<int, 2>{}); break;
    case 3: run(std::integral_constant<int, 3>{}); break;
    case 4: run(std::integral_constant<int, 4>{}); break;
    default: {
      // this wave row holds no valid row: make its copies and keep the
      // barrier count of the others
      const std::integral_constant<int, 0> none{};
      prologue(none);
      int kt = 0;
      auto idle_step = [&](auto uc, int k) {  // step k of a wave row without MFMA work
        constexpr int u = decltype(uc)::value;
        if (SPREAD && k + NB - 1 < nk) issueB(b_slot((u + NB - 1) % NB), k + NB - 1);
        handover(none, uc, k, std::false_type{});
      };
      for (; kt + 6 < nk; kt += 6)
        unroll<6>([&](auto uc) { idle_step(uc, kt + decltype(uc)::value); });
      for (; kt + 1 < nk; kt += 6)
        unroll<6>([&](auto uc) {
          if (kt + decltype(uc)::value + 1 < nk) idle_step(uc, kt + decltype(uc)::value);
        });
    }
  }

  // epilogue scratch in the slots (no copy is in flight any more): hidden
  // blocks in slot 0, the row table in slot 1, fp32 blocks in slots 2 and 3
  tile_epilogue<C, MODE, true, true>(
      gu, dn, acc, g, row0, rows, col0, kc, wrow0, live_m, row_a, row_wt, ls0 + wave * (MB * HC),
      reinterpret_cast<float*>(wave < NW / 2 ? ls2 : ls3) + (wave % (NW / 2)) * (MB * TN),
      reinterpret_cast<int*>(ls1), reinterpret_cast<float*>(ls1) + BM);
}

// out[t][d] = Y[t][k][d] + Y[t][0][d] + ... + Y[t][k-1][d] (+ residual[t][d]),
// four columns per thread.  KC > 0 fixes k at compile time, so every slot's
// load is issued before the first add; KC = 0 takes k at run time.  The slot
// rows are read once: non-temporal loads.
template <int RES, int KC>  // RES 0: none, 1: bf16 residual, 2: fp32 residual
__global__ __launch_bounds__(256) void combine_kernel(const float* __restrict__ Y,
                                                      float* __restrict__ out, int T, int D,
                                                      int k_rt, const void* __restrict__ residual) {
  const int k = KC > 0 ? KC : k_rt;
  const int D4 = D / 4;
  const size_t i = (size_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= (size_t)T * D4) return;
  const int t = (int)(i / D4), c = (int)(i % D4);
  const f32x4* y = reinterpret_cast<const f32x4*>(Y + (size_t)t * (k + 1) * D) + c;
  const f32x4 vs = __builtin_nontemporal_load(y + (size_t)k * D4);
  float4 v = make_float4(vs.x, vs.y, vs.z, vs.w);
  if constexpr (KC > 0) {
    f32x4 u[KC];
#pragma unroll
    for (int j = 0; j < KC; ++j) u[j] = __builtin_nontemporal_load(y + (size_t)j * D4);
#pragma unroll
    for (int j = 0; j < KC; ++j) {
      v.x += u[j].x; v.y += u[j].y; v.z += u[j].z; v.w += u[j].w;
    }
  } else {
    // four slots' loads in flight at a time; the adds stay in slot order
    int j = 0;
    for (; j + 4 <= k; j += 4) {
      f32x4 u[4];
#pragma unroll
      for (int q = 0; q < 4; ++q) u[q] = __builtin_nontemporal_load(y + (size_t)(j + q) * D4);
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        v.x += u[q].x; v.y += u[q].y; v.z += u[q].z; v.w += u[q].w;
      }
    }
    for (; j < k; ++j) {
      const f32x4 u = __builtin_nontemporal_load(y + (size_t)j * D4);
      v.x += u.x; v.y += u.y; v.z += u.z; v.w += u.w;
    }
  }
  if constexpr (RES == 1) {
    const uint2 r = reinterpret_cast<const uint2*>(static_cast<const bf16_t*>(residual) +
                                                   (size_t)t * D)[c];
    v.x += __uint_as_float(r.x << 16); v.y += __uint_as_float(r.x & 0xFFFF0000u);
    v.z += __uint_as_float(r.y << 16); v.w += __uint_as_float(r.y & 0xFFFF0000u);
  } else if constexpr (RES == 2) {
    const float4 r = reinterpret_cast<const float4*>(static_cast<const float*>(residual) +
                                                     (size_t)t * D)[c];
    v.x += r.x; v.y += r.y; v.z += r.z; v.w += r.w;
  }
  reinterpret_cast<float4*>(out + (size_t)t * D)[c] = v;
}

// Tile configurations: <BM, BN, BK, WM, WN, stages, MFMA block>.
#ifndef GLM_CFG_DECODE
#define GLM_CFG_DECODE 32, 128, 64, 1, 4, 5, 16
#endif
using CfgDecode = Cfg<GLM_CFG_DECODE>;  // few rows per expert: weight streaming
#ifndef GLM_CFG_MID
#define GLM_CFG_MID 128, 256, 64, 2, 4, 3, 32
#endif
using CfgMid = Cfg<GLM_CFG_MID>;
#ifndef GLM_CFG_BIG
#define GLM_CFG_BIG 256, 256, 64, 2, 4, 2, 32
#endif
using CfgBig = Cfg<GLM_CFG_BIG>;  // prefill: 8 waves (two per SIMD), BK 64, 2 stages
using CfgNarrow = Cfg<32, 64, 64, 1, 2, 4, 16>;    // widths that are not a multiple of 128/256
// a dense layer on 33..96 tokens: one row tile up to 64 tokens, so each
// weight slice is streamed by one workgroup
#ifndef GLM_CFG_DECODE64
#define GLM_CFG_DECODE64 64, 128, 64, 1, 4, 5, 16
#endif
using CfgDecode64 = Cfg<GLM_CFG_DECODE64>;

#ifndef GLM_SPLIT_BIG
#define GLM_SPLIT_BIG 1
#endif
#ifndef GLM_SPLIT_NA  // activation slots of the split rings (the weight ring has the rest of 5)
#define GLM_SPLIT_NA 2
#endif
template <class C, int MODE>
hipError_t launch_one(const GateUpArgs& gu, const DownArgs& dn, unsigned grid, hipStream_t s) {
  if (grid == 0) return hipSuccess;
  if constexpr (C::BM == 256 && C::BN == 256 && C::BK == 64 && C::MB == 32 && GLM_SPLIT_BIG) {
    split_gemm_kernel<C, MODE, GLM_SPLIT_NA, 5 - GLM_SPLIT_NA><<<grid, C::NT, 0, s>>>(gu, dn);
    return hipGetLastError();
  }
  if constexpr (C::ST == 2) {
    if (MODE == GATE_UP ? gu.early : dn.early) {
      grouped_gemm_kernel<C, MODE, true><<<grid, C::NT, 0, s>>>(gu, dn);
      return hipGetLastError();
    }
  }
  grouped_gemm_kernel<C, MODE, false><<<grid, C::NT, 0, s>>>(gu, dn);
  return hipGetLastError();
}

template <int MODE>
hipError_t dispatch(GemmShape sh, const GateUpArgs& gu, const DownArgs& dn, unsigned grid,
                    hipStream_t s) {
  if (sh.BM == CfgDecode::BM && sh.BN == CfgDecode::BN)
    return launch_one<CfgDecode, MODE>(gu, dn, grid, s);
  if (sh.BM == CfgMid::BM && sh.BN == CfgMid::BN) return launch_one<CfgMid, MODE>(gu, dn, grid, s);
  if (sh.BM == CfgBig::BM && sh.BN == CfgBig::BN) return launch_one<CfgBig, MODE>(gu, dn, grid, s);
  if (sh.BM == CfgNarrow::BM && sh.BN == CfgNarrow::BN)
    return launch_one<CfgNarrow, MODE>(gu, dn, grid, s);
  if (sh.BM == CfgDecode64::BM && sh.BN == CfgDecode64::BN)
    return launch_one<CfgDecode64, MODE>(gu, dn, grid, s);
  return hipErrorInvalidValue;
}

}  // namespace gemm

using namespace gemm;

GemmShape gemm_shape(double rows_per_group, bool wide) {
  if (!wide) return {CfgNarrow::BM, CfgNarrow::BN};
  if (rows_per_group <= 24.0) return {CfgDecode::BM, CfgDecode::BN};
#ifndef GLM_MID_MAX_ROWS
#define GLM_MID_MAX_ROWS 96.0
#endif
  if (rows_per_group <= GLM_MID_MAX_ROWS) return {CfgMid::BM, CfgMid::BN};
  return {CfgBig::BM, CfgBig::BN};
}

// Workgroups of the config with tile shape `sh` that fit on one CU at once
// (LDS: the stage ring; 160 KB per CU).
template <class C>
constexpr int wgs_per_cu() {
  return (160 * 1024) / (C::ST * C::STAGE * 2 + C::BM * 8);
}
int gemm_wgs_per_cu(GemmShape sh) {
  if (sh.BM == CfgDecode::BM && sh.BN == CfgDecode::BN) return wgs_per_cu<CfgDecode>();
  if (sh.BM == CfgDecode64::BM && sh.BN == CfgDecode64::BN) return wgs_per_cu<CfgDecode64>();
  if (sh.BM == CfgNarrow::BM && sh.BN == CfgNarrow::BN) return wgs_per_cu<CfgNarrow>();
  if (sh.BM == CfgMid::BM && sh.BN == CfgMid::BN) return wgs_per_cu<CfgMid>();
  return 1;
}

GemmShape gemm_shape_few(int rows, bool wide) {
  if (!wide) return {CfgNarrow::BM, CfgNarrow::BN};
  if (rows <= CfgDecode::BM) return {CfgDecode::BM, CfgDecode::BN};
  return {CfgDecode64::BM, CfgDecode64::BN};
}

hipError_t launch_gateup_bf16(const GateUpArgs& a, GemmShape sh, hipStream_t s) {
  return dispatch<GATE_UP>(sh, a, DownArgs{}, (unsigned)a.grid, s);
}

hipError_t launch_down_bf16(const DownArgs& a, GemmShape sh, hipStream_t s) {
  return dispatch<DOWN>(sh, GateUpArgs{}, a, (unsigned)a.grid, s);
}

namespace {
__global__ __launch_bounds__(256) void gateup_fixup_kernel(const float* __restrict__ P,
                                                           bf16_t* __restrict__ Hs, int T, int Fs,
                                                           int c0, int w, int ks) {
  const int W4 = w / 4;
  const size_t i = (size_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= (size_t)T * W4) return;
  const int t = (int)(i / W4), c = (int)(i % W4) * 4;
  f32x4 g = {0.f, 0.f, 0.f, 0.f}, u = {0.f, 0.f, 0.f, 0.f};
  for (int kc = 0; kc < ks; ++kc) {
    const float* p = P + ((size_t)kc * T + t) * (2 * w);
    g += __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(p + c));
    u += __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(p + w + c));
  }
  bf16_t h[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) h[j] = f32_to_bf16(silu(g[j]) * u[j]);
  *reinterpret_cast<uint2*>(Hs + (size_t)t * Fs + c0 + c) =
      make_uint2((uint32_t)h[0] | ((uint32_t)h[1] << 16), (uint32_t)h[2] | ((uint32_t)h[3] << 16));
}
}  // namespace

hipError_t launch_gateup_fixup(const float* P, bf16_t* Hs, int T, int Fs, int c0, int w, int ks,
                               hipStream_t s) {
  const size_t n = (size_t)T * (w / 4);
  if (n == 0) return hipSuccess;
  gateup_fixup_kernel<<<(unsigned)((n + 255) / 256), 256, 0, s>>>(P, Hs, T, Fs, c0, w, ks);
  return hipGetLastError();
}

hipError_t launch_combine(const float* Y, float* out, int T, int D, int k, const void* residual,
                          bool res_bf16, hipStream_t s) {
  const size_t n = (size_t)T * (D / 4);
  if (n == 0) return hipSuccess;
  const unsigned grid = (unsigned)((n + 255) / 256);
  if (k == 8) {
    if (!residual) combine_kernel<0, 8><<<grid, 256, 0, s>>>(Y, out, T, D, k, nullptr);
    else if (res_bf16) combine_kernel<1, 8><<<grid, 256, 0, s>>>(Y, out, T, D, k, residual);
    else combine_kernel<2, 8><<<grid, 256, 0, s>>>(Y, out, T, D, k, residual);
  } else {
    if (!residual) combine_kernel<0, 0><<<grid, 256, 0, s>>>(Y, out, T, D, k, nullptr);
    else if (res_bf16) combine_kernel<1, 0><<<grid, 256, 0, s>>>(Y, out, T, D, k, residual);
    else combine_kernel<2, 0><<<grid, 256, 0, s>>>(Y, out, T, D, k, residual);
  }
  return hipGetLastError();
}

}  // namespace glm
