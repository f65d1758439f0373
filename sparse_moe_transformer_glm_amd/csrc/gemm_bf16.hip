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



// EARLY (two stages only): each stage's refill is issued before the wait for
// the next stage instead of after it (see the main loop).
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
  int g = 0, row0 = 0, rows = 0, col0 = 0, K = 0;
  bool sole = false;
  if constexpr (MODE == GATE_UP) {
    const int i = xcd_tile(*gu.desc_count, gu.xblk);
    if (i < 0) return;
    const TileDesc d = gu.desc[i];
    g = d.group & kGroupMask; sole = d.group & kSoleRowTile; row0 = d.row0; rows = d.rows;
    col0 = d.col0; K = gu.D;
  } else {
    const int i = xcd_tile(*dn.desc_count, dn.xblk);
    if (i < 0) return;
    const TileDesc d = dn.desc[i];
    g = d.group & kGroupMask; sole = d.group & kSoleRowTile; row0 = d.row0; rows = d.rows;
    col0 = d.col0;
    K = (g == dn.E) ? dn.Fs : dn.F;
  }

  // DMA sources: instruction q = wave + i*NW covers rows [q*RPI, q*RPI+RPI) of
  // the stage (A rows first, then B rows); lane l fills physical chunk l % CPR
  // of row q*RPI + l / CPR, i.e. logical chunk (l % CPR) ^ swz(row).
  const bf16_t* src[IPW];
#pragma unroll
  for (int i = 0; i < IPW; ++i) {
    const int q = wave + i * NW;
    const int r = q * RPI + lane / CPR;
    const int ch = (lane % CPR) ^ swz<BK>(r);
    const bf16_t* base;
    if (r < BM) {
      const int rr = min(r, rows - 1);  // rows past the tile repeat its last row
      if constexpr (MODE == GATE_UP) {
        const int tok = (g == gu.E) ? row0 + rr
                                    : gu.row_assign[row0 + rr] / gu.k;
        base = gu.x + (size_t)tok * gu.D;
      } else {
        base = (g == dn.E) ? dn.Hs + (size_t)(row0 + rr) * dn.Fs
                           : dn.H + (size_t)(row0 + rr) * dn.F;
      }
    } else {
      const int n = r - BM;
      if constexpr (MODE == GATE_UP) {
        const int blk = n / MB, hcol = col0 + (blk / 2) * MB + (n % MB);
        const bool up = blk & 1;
        if (g == gu.E) base = (up ? gu.sw3 : gu.sw1) + (size_t)hcol * gu.D;
        else base = (up ? gu.w3 : gu.w1) + ((size_t)g * gu.F + hcol) * gu.D;
      } else {
        base = (g == dn.E) ? dn.sw2 + (size_t)(col0 + n) * dn.Fs
                           : dn.w2 + ((size_t)g * dn.D + col0 + n) * dn.F;
      }
    }
    src[i] = base + ch * 8;
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

  // rows of this tile handled by each wave row: an even split in MB blocks
  const int per = min(TM, ((rows + C::WM - 1) / C::WM + MB - 1) / MB * MB);
  const int wrow0 = wm * per;
  const int live_m = min(min(FM, per / MB), max(0, (rows - wrow0 + MB - 1) / MB));

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
      if (s < nk) issue(stage_ptr(s), s, nt_c);
    if (ST - 1 < nk) __builtin_amdgcn_s_waitcnt(GLM_VMCNT(IPW * (ST - 1)));
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
              issue(cur, kt + 2, nt_c);
              __builtin_amdgcn_s_waitcnt(GLM_VMCNT(IPW));  // this wave's copies of kt+1
            } else {
              __builtin_amdgcn_s_waitcnt(GLM_VMCNT(0));
            }
            asm volatile("s_barrier" ::: "memory");
          } else {
            if (kt + ST - 1 < nk) __builtin_amdgcn_s_waitcnt(GLM_VMCNT(IPW * (ST - 2)));
            else __builtin_amdgcn_s_waitcnt(GLM_VMCNT(0));
            lds_barrier();
            if (kt + ST < nk) issue(cur, kt + ST, nt_c);
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
        // this wave row holds no valid row: keep the barrier count of the others
        for (int s = 0; s < ST; ++s)
          if (s < nk) issue(stage_ptr(s), s, nt_c);
        __builtin_amdgcn_s_waitcnt(GLM_VMCNT(0));
        lds_barrier();
        for (int kt = 0; kt + 1 < nk; ++kt) {
          if constexpr (early) {  // the same two barriers per step as the other waves
            lds_barrier();
            if (kt + 2 < nk) {
              issue(stage_ptr(kt % ST), kt + 2, nt_c);
              __builtin_amdgcn_s_waitcnt(GLM_VMCNT(IPW));
            } else {
              __builtin_amdgcn_s_waitcnt(GLM_VMCNT(0));
            }
            asm volatile("s_barrier" ::: "memory");
          } else {
            __builtin_amdgcn_s_waitcnt(GLM_VMCNT(0));
            lds_barrier();
            if (kt + ST < nk) issue(stage_ptr(kt % ST), kt + ST, nt_c);
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
    if constexpr (NW * MB * HC * 2 <= C::STAGE * 2 && HC % 8 == 0 &&
                  MB % (kWave / (HC / 8 > 0 ? HC / 8 : 1)) == 0) {
      // Through LDS, one MB-row block at a time (as the down epilogue):
      // 16-byte stores of 8 consecutive hidden values.
      bf16_t* blk = lds0 + wave * (MB * HC);
      constexpr int CG = HC / 8, RPP = kWave / CG;
      static_assert(kWave % CG == 0 && MB % RPP == 0, "epilogue pass shape");
      const int hcol0 = col0 + wn * HC;
      __syncthreads();  // every wave is done reading the stages
#pragma unroll
      for (int m = 0; m < FM; ++m) {
        if (m >= live_m) continue;
#pragma unroll
        for (int q = 0; q < FN / 2; ++q)
#pragma unroll
          for (int r = 0; r < NR; ++r) {
            const int rb = row_of(m, r) - (wrow0 + m * MB);
            const float h = silu(acc[m][2 * q][r]) * acc[m][2 * q + 1][r];
            blk[rb * HC + q * MB + lr] = f32_to_bf16(h);
          }
#pragma unroll
        for (int pass = 0; pass < MB / RPP; ++pass) {
          const int rb = pass * RPP + lane / CG, cg = lane % CG;
          const int row = wrow0 + m * MB + rb;
          const uint4 v = *reinterpret_cast<const uint4*>(blk + rb * HC + 8 * cg);
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
    // row of Y and routing weight of every row of the tile
    if (tid < rows) {
      s_asg[tid] = g == dn.E ? (row0 + tid) * (dn.k + 1) + dn.k : y_row(row_a, dn.k);
      s_wt[tid] = row_wt;
    }
    __syncthreads();  // the row table is complete and every wave is done reading the stages
    if constexpr (NW * MB * TN * 4 <= C::STAGE * 2) {
      // Through LDS, one MB-row block at a time: each wave writes its block
      // (MB x TN fp32) to its own slice of stage 0, then stores whole 16-byte
      // column groups, so a store instruction covers a few full row pieces.
      float* blk = reinterpret_cast<float*>(lds0) + wave * (MB * TN);
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
          for (int n = 0; n < FN; ++n) blk[rb * TN + n * MB + lr] = acc[m][n][r];
        }
#pragma unroll
        for (int pass = 0; pass < MB / RPP; ++pass) {
          const int rb = pass * RPP + lane / CG, cg = lane % CG;
          const int row = wrow0 + m * MB + rb;
          const float4 v = *reinterpret_cast<const float4*>(blk + rb * TN + 4 * cg);
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
    for (int j = 0; j < k; ++j) {
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

template <class C, int MODE>
hipError_t launch_one(const GateUpArgs& gu, const DownArgs& dn, unsigned grid, hipStream_t s) {
  if (grid == 0) return hipSuccess;
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

hipError_t launch_gateup_bf16(const GateUpArgs& a, GemmShape sh, hipStream_t s) {
  return dispatch<GATE_UP>(sh, a, DownArgs{}, (unsigned)a.grid, s);
}

hipError_t launch_down_bf16(const DownArgs& a, GemmShape sh, hipStream_t s) {
  return dispatch<DOWN>(sh, GateUpArgs{}, a, (unsigned)a.grid, s);
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
