// MXFP8 grouped expert GEMMs of the GLM-5.2 MoE layer on gfx950's
// block-scaled FP8 MFMA (v_mfma_scale_f32_32x32x64_f8f6f4).
//
// Format: OCP MX with E4M3 elements and one E8M0 scale per 32 consecutive
// elements along the contraction dimension.  The pages name BF16/FP8 GLM-5.2
// artifacts ("Inside GLM" course page, Release anatomy lesson) but
// not their scaling; MX is the format this hardware scales inside the MFMA.
//
// Same data flow as the bf16 kernels: C[M x N] = A[M x K] . B[N x K]^T, both
// operands K-contiguous, one workgroup per BM x BN tile from the device-built
// tile list, K walked in steps of 128 elements (bytes) through a ring of LDS
// stages filled by 16-byte LDS-DMA loads.  Each stage also holds the tile's
// E8M0 scales for the step (4 per row, one dword), loaded by 4-byte LDS-DMA.
//
// Scales are stored K-step-major: the four scales of row n for K step kt
// (elements [128kt, 128kt+128)) are the dword at (kt * N + n) * 4 of the
// matrix's scale array (N rows), so the 64 rows of one scale copy are 256
// contiguous bytes.  The weights arrive in this layout (the pack entry point
// converts from row-major scales); the quantised activations and hidden rows
// are written in it.
//
// MFMA operand layout (checked on gfx950): lane l supplies row l % 32; with
// g = l / 32 its 32 bytes are K elements [16g, 16g+16) and [32+16g, 32+16g+16)
// of the 64-element step, and the scale it passes covers K elements
// [32g, 32g+32) of both lane groups.  So lane group g reads the two 16-byte
// chunks g and g+2 of each 64-byte half-step and passes the scale of MX block
// 2 * sub + g; with that, the hardware's K blocks are exactly the tensors'.
//
// Epilogues: GATE_UP forms h = SiLU(g) * u in fp32 and quantises it to MXFP8
// along the hidden dimension (a 32-column MFMA block is one MX block: the
// block maximum is a 32-lane reduction), writing codes and scales for the
// down projection.  DOWN writes w * (H W2^T) in fp32 to its (token, slot) row
// of Y, exactly as the bf16 kernel, and the shared combine follows unchanged.
#include "common.h"

#include <type_traits>

namespace glm {
namespace gemm_mx {

enum Mode { GATE_UP = 0, DOWN = 1 };

typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int BK = 128;   // K elements (bytes) per stage
constexpr int KSUB = 2;   // 64-element MFMA steps per stage
constexpr int CPR = 8;    // 16-byte chunks per row
constexpr int RPI = 8;    // rows per 1 KB DMA instruction
#ifndef GLM_MX_LIVE_A  // copy only the live row blocks' activation rows
#define GLM_MX_LIVE_A 1
#endif

template <int BM_, int BN_, int WM_, int WN_, int ST_>
struct Cfg {
  static constexpr int BM = BM_, BN = BN_, WM = WM_, WN = WN_, ST = ST_;
  static constexpr int NW = WM * WN, NT = NW * kWave;
  static constexpr int TM = BM / WM, TN = BN / WN;
  static constexpr int FM = TM / 32, FN = TN / 32;
  static constexpr int A_INST = BM / RPI, B_INST = BN / RPI;
  static constexpr int IPW = (A_INST + B_INST) / NW;  // data DMAs per wave per stage
  // scale DMAs: 64 rows (one dword each) per instruction
  static constexpr int SA_INST = (BM + 63) / 64, SB_INST = BN / 64;
  static constexpr int S_INST = SA_INST + SB_INST;
  static constexpr int SPW = (S_INST + NW - 1) / NW;  // scale DMAs per wave per stage
  static constexpr int SC_A = (BM + BN) * BK;         // byte offset of the A scales
  static constexpr int SC_B = SC_A + SA_INST * 256;   // byte offset of the B scales
  static constexpr int STAGE = SC_B + SB_INST * 256;  // bytes per stage
  static_assert(TM % 32 == 0 && TN % 64 == 0, "wave tile: whole 32-row blocks, gate/up pairs");
  static_assert(BM % RPI == 0 && BN % 64 == 0, "tiles must be whole DMA instructions");
  static_assert((A_INST + B_INST) % NW == 0, "every wave issues the same number of DMAs");
  static_assert(A_INST % NW == 0, "copy i of every wave is an A copy exactly when i < A_INST / NW");
  static_assert(FM <= 4, "live-block dispatch covers up to 4 row blocks");
  static_assert(ST >= 2 && ST <= 8, "ring of 2 to 8 stages");
};

// Physical 16-byte chunk of logical chunk c of row r (8 chunks per row):
// rows r..r+15 reading one logical chunk hit distinct LDS banks.
__device__ __forceinline__ int swz(int r) { return (r & 7) ^ ((r >> 3) & 1); }

__device__ inline float silu(float g) { return g / (1.0f + expf(-g)); }


// Smallest s with amax <= 448 * 2^s (0 for amax == 0): with amax = f * 2^x,
// f in [0.5, 1), it is x - 9 when f <= 0.875, else x - 8.
__device__ __forceinline__ int mx_exponent(float amax) {
  int x;
  const float f = frexpf(amax, &x);
  // (the lower clamp keeps the E8M0 code valid for blocks below 2^-118,
  // which hold only fp32 subnormals)
  return amax == 0.0f ? 0 : max(f <= 0.875f ? x - 9 : x - 8, -127);
}

// Nearest E4M3 code (ties to even) of |y| <= 448: integer rounding of the
// fp32 pattern to 3 mantissa bits for results from 2^-6 up, rounding of
// y * 2^9 below (the subnormal step is 2^-9; codes are contiguous there).
__device__ __forceinline__ uint32_t e4m3_code(float y) {
  const uint32_t u = __float_as_uint(y) & 0x7FFFFFFFu;
  uint32_t c;
  if (u >= ((127u - 6u) << 23)) {
    c = ((u + 0x7FFFFu + ((u >> 20) & 1u)) >> 20) - ((127u - 7u) << 3);
  } else {
    c = (uint32_t)rintf(__uint_as_float(u) * 512.0f);
  }
  const bool neg = (__float_as_uint(y) >> 31) && u != 0;
  return c | (neg ? 0x80u : 0u);
}


template <class C, int MODE>
__global__ __launch_bounds__(C::NT) void grouped_gemm_mx_kernel(MxGateUpArgs gu, MxDownArgs dn) {
  constexpr int BM = C::BM, BN = C::BN, ST = C::ST;
  constexpr int WN = C::WN, NW = C::NW, TM = C::TM, TN = C::TN, FM = C::FM, FN = C::FN;
  constexpr int IPW = C::IPW, SPW = C::SPW;

  __shared__ __attribute__((aligned(1024))) uint8_t lds0[C::STAGE];
  __shared__ __attribute__((aligned(1024))) uint8_t lds1[C::STAGE];
  __shared__ __attribute__((aligned(1024))) uint8_t lds2[ST > 2 ? C::STAGE : 16];
  __shared__ __attribute__((aligned(1024))) uint8_t lds3[ST > 3 ? C::STAGE : 16];
  __shared__ __attribute__((aligned(1024))) uint8_t lds4[ST > 4 ? C::STAGE : 16];
  __shared__ __attribute__((aligned(1024))) uint8_t lds5[ST > 5 ? C::STAGE : 16];
  __shared__ __attribute__((aligned(1024))) uint8_t lds6[ST > 6 ? C::STAGE : 16];
  __shared__ __attribute__((aligned(1024))) uint8_t lds7[ST > 7 ? C::STAGE : 16];
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
  const int KS = K / 32;  // scale bytes per row

  // Data row and K-step-0 scale dword of A (tile row rr) and B (tile column
  // n); *sstep is the byte distance between K steps of that scale array.
  auto a_row = [&](int rr, const uint8_t** data, const uint8_t** sc, size_t* sstep) {
    rr = min(rr, rows - 1);  // rows past the tile repeat its last row
    if constexpr (MODE == GATE_UP) {
      if (g == gu.E) {
        *data = gu.xq + (size_t)(row0 + rr) * K;
        *sc = gu.xs + (size_t)(row0 + rr) * 4;
        *sstep = (size_t)gu.T * 4;
      } else {
        const int r = row0 + rr;
        *data = gu.xq + (size_t)(gu.row_assign[r] / gu.k) * K;
        *sc = gu.xsp + (size_t)r * 4;
        *sstep = (size_t)gu.T * gu.k * 4;
      }
    } else if (g == dn.E) {
      *data = dn.Hs + (size_t)(row0 + rr) * K;
      *sc = dn.Hssc + (size_t)(row0 + rr) * 4;
      *sstep = (size_t)dn.T * 4;
    } else {
      const size_t r = (size_t)(row0 + rr);
      *data = dn.H + r * K;
      *sc = dn.Hsc + r * 4;
      *sstep = (size_t)dn.T * dn.k * 4;
    }
  };
  auto b_row = [&](int n, const uint8_t** data, const uint8_t** sc, size_t* sstep) {
    if constexpr (MODE == GATE_UP) {
      const int blk = n / 32, hcol = col0 + (blk / 2) * 32 + (n % 32);
      const bool up = blk & 1;
      if (g == gu.E) {
        *data = (up ? gu.sw3 : gu.sw1) + (size_t)hcol * K;
        *sc = (up ? gu.sw3s : gu.sw1s) + (size_t)hcol * 4;
        *sstep = (size_t)gu.Fs * 4;
      } else {
        const size_t r = (size_t)g * gu.F + hcol;
        *data = (up ? gu.w3 : gu.w1) + r * K;
        *sc = (up ? gu.w3s : gu.w1s) + (size_t)g * gu.F * KS + (size_t)hcol * 4;
        *sstep = (size_t)gu.F * 4;
      }
    } else if (g == dn.E) {
      *data = dn.sw2 + (size_t)(col0 + n) * K;
      *sc = dn.sw2s + (size_t)(col0 + n) * 4;
      *sstep = (size_t)dn.D * 4;
    } else {
      *data = dn.w2 + ((size_t)g * dn.D + col0 + n) * K;
      *sc = dn.w2s + (size_t)g * dn.D * KS + (size_t)(col0 + n) * 4;
      *sstep = (size_t)dn.D * 4;
    }
  };

  // DMA sources.  Data instruction q = wave + i*NW covers 8 rows (A rows
  // first, then B rows); lane l fills physical chunk l % 8 of row q*8 + l/8.
  const uint8_t* src[IPW];
#pragma unroll
  for (int i = 0; i < IPW; ++i) {
    const int q = wave + i * NW;
    const int r = q * RPI + lane / CPR;
    const int ch = (lane % CPR) ^ swz(r);
    const uint8_t* d;
    const uint8_t* sc;
    size_t step;
    if (r < BM) a_row(r, &d, &sc, &step);
    else b_row(r - BM, &d, &sc, &step);
    src[i] = d + ch * 16;
  }
  // Scale instruction j covers 64 rows: j < SA_INST the A rows, else B rows.
  // Waves beyond the instruction count repeat instruction j % S_INST (the
  // same bytes to the same place).
  const uint8_t* ssrc[SPW];
  size_t sstep[SPW];
  int sdst[SPW];
#pragma unroll
  for (int i = 0; i < SPW; ++i) {
    const int j = (wave + i * NW) % C::S_INST;
    const uint8_t* d;
    if (j < C::SA_INST) {
      a_row(j * 64 + lane, &d, &ssrc[i], &sstep[i]);
      sdst[i] = C::SC_A + j * 256;
    } else {
      b_row((j - C::SA_INST) * 64 + lane, &d, &ssrc[i], &sstep[i]);
      sdst[i] = C::SC_B + (j - C::SA_INST) * 256;
    }
  }

  // 32-row MFMA blocks holding valid rows, dealt to the wave rows as evenly
  // as possible (a SIMD runs one wave of each wave row)
  const int nb = (rows + 31) / 32;
  const int live_m = min(FM, nb / C::WM + (wm < nb % C::WM ? 1 : 0));
  const int wrow0 = 32 * (wm * (nb / C::WM) + min(wm, nb % C::WM));

  // LIVEA: instead of the uniform data copies above, copy c of wave (wm, wn)
  // fills rows (c*WN + wn)*RPI .. +RPI of each live row block of its wave row
  // (CPB copies a block), so rows of blocks past the valid rows are never
  // fetched (their LDS rows reach no MFMA); B copy i covers B rows
  // (wave + i*NW)*RPI .. +RPI.  The scale copies stay as above.
  constexpr int CPB = 32 / (WN * RPI) > 0 ? 32 / (WN * RPI) : 1;
  constexpr bool LIVEA = GLM_MX_LIVE_A && CPB * WN * RPI == 32 && C::B_INST % NW == 0;
  constexpr int BW = C::B_INST / NW;
  const uint8_t* sa_l[LIVEA ? FM * CPB : 1];
  int a_dst[LIVEA ? FM * CPB : 1];
  const uint8_t* sb_l[LIVEA ? BW : 1];
  if constexpr (LIVEA) {
#pragma unroll
    for (int i = 0; i < FM * CPB; ++i) {
      a_dst[i] = min(wrow0 + (i / CPB) * 32, BM - 32) + ((i % CPB) * WN + wn) * RPI;
      const int r = a_dst[i] + lane / CPR;
      const uint8_t* d;
      const uint8_t* sc;
      size_t step;
      a_row(r, &d, &sc, &step);
      sa_l[i] = d + ((lane % CPR) ^ swz(r)) * 16;
    }
#pragma unroll
    for (int i = 0; i < BW; ++i) {
      const int n = (wave + i * NW) * RPI + lane / CPR;
      const uint8_t* d;
      const uint8_t* sc;
      size_t step;
      b_row(n, &d, &sc, &step);
      sb_l[i] = d + ((lane % CPR) ^ swz(BM + n)) * 16;
    }
  }

  // Per-row data of the down epilogue, loaded into registers here and written
  // to LDS at the epilogue (the loads stay off the path to the first K step).
  static_assert(BM <= C::NT, "one epilogue row per thread");
  int row_a = 0;
  float row_wt = 1.0f;
  if constexpr (MODE == DOWN) {
    if (tid < rows && g != dn.E) {
      row_a = dn.row_assign[row0 + tid];
      row_wt = dn.row_w[row0 + tid];
    }
  }

  auto stage_ptr = [&](int s) -> uint8_t* {
    return s == 0 ? lds0 : s == 1 ? lds1 : s == 2 ? lds2 : s == 3 ? lds3
         : s == 4 ? lds4 : s == 5 ? lds5 : s == 6 ? lds6 : lds7;
  };
  // NT: weight rows go with the non-temporal hint (a sole row tile, see kStreamB)
  auto issue = [&](uint8_t* st, int kt, auto nt_c) {
    constexpr bool NT = decltype(nt_c)::value;
#pragma unroll
    for (int i = 0; i < IPW; ++i) {
      const int q = wave + i * NW;
      if (NT && i * NW >= C::A_INST)  // a weight-row copy
        __builtin_amdgcn_global_load_lds((const void*)(src[i] + (size_t)kt * BK),
                                         (lds_void*)(st + q * (RPI * BK)), 16, 0, kCpolNt);
      else
        __builtin_amdgcn_global_load_lds((const void*)(src[i] + (size_t)kt * BK),
                                         (lds_void*)(st + q * (RPI * BK)), 16, 0, 0);
    }
#pragma unroll
    for (int i = 0; i < SPW; ++i)
      __builtin_amdgcn_global_load_lds((const void*)(ssrc[i] + (size_t)kt * sstep[i]),
                                       (lds_void*)(st + sdst[i]), 4, 0, 0);
  };
  // copies of step kt into stage st: LIVE * CPB A copies, BW B copies and the
  // scale copies (LIVEA), else the uniform ones
  auto issue_any = [&](uint8_t* st, int kt, auto nt_c, auto live_c) {
    if constexpr (LIVEA) {
      constexpr bool NT = decltype(nt_c)::value;
      constexpr int LIVE = decltype(live_c)::value;
#pragma unroll
      for (int i = 0; i < LIVE * CPB; ++i)
        __builtin_amdgcn_global_load_lds((const void*)(sa_l[i] + (size_t)kt * BK),
                                         (lds_void*)(st + a_dst[i] * BK), 16, 0, 0);
#pragma unroll
      for (int i = 0; i < BW; ++i)
        __builtin_amdgcn_global_load_lds((const void*)(sb_l[i] + (size_t)kt * BK),
                                         (lds_void*)(st + (BM + (wave + i * NW) * RPI) * BK),
                                         16, 0, NT ? kCpolNt : 0);
#pragma unroll
      for (int i = 0; i < SPW; ++i)
        __builtin_amdgcn_global_load_lds((const void*)(ssrc[i] + (size_t)kt * sstep[i]),
                                         (lds_void*)(st + sdst[i]), 4, 0, 0);
    } else {
      issue(st, kt, nt_c);
    }
  };

  const int lr = lane % 32, lg = lane / 32;
  const int sw = swz(lr);

  f32x16 acc[FM][FN];
#pragma unroll
  for (int m = 0; m < FM; ++m)
#pragma unroll
    for (int n = 0; n < FN; ++n) acc[m][n] = f32x16{};

  const int nk = K / BK;

  // LDS byte offsets of this lane's fragment chunks: row base plus the
  // swizzled chunk of (sub-step, half); rows 32 apart share the swizzle, so
  // the m / n blocks are constant offsets of 32 rows (4 KB) from these.
  const int a_row0 = (wrow0 + lr) * BK, b_row0 = (BM + wn * TN + lr) * BK;
  int coff[KSUB][2];
#pragma unroll
  for (int sub = 0; sub < KSUB; ++sub)
#pragma unroll
    for (int h = 0; h < 2; ++h) coff[sub][h] = ((4 * sub + 2 * h + lg) ^ sw) * 16;
  const int a_sc = C::SC_A + (wrow0 + lr) * 4, b_sc = C::SC_B + (wn * TN + lr) * 4;

  auto run = [&](auto live_c, auto nt_c) {
    constexpr int LIVE = decltype(live_c)::value;
    constexpr int VPS = LIVEA ? LIVE * CPB + BW + SPW : IPW + SPW;  // copies per wave and stage
    i32x8 fa[LIVE > 0 ? LIVE : 1], fb[FN];
    uint32_t sa[LIVE > 0 ? LIVE : 1], sb[FN];
    auto frag = [&](const uint8_t* st, int lo_off, int hi_off) -> i32x8 {
      const i32x4 lo = *reinterpret_cast<const i32x4*>(st + lo_off);
      const i32x4 hi = *reinterpret_cast<const i32x4*>(st + hi_off);
      return i32x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
    };
    auto load_scales = [&](const uint8_t* st) {
#pragma unroll
      for (int m = 0; m < LIVE; ++m)
        sa[m] = *reinterpret_cast<const uint32_t*>(st + a_sc + m * 32 * 4);
#pragma unroll
      for (int n = 0; n < FN; ++n)
        sb[n] = *reinterpret_cast<const uint32_t*>(st + b_sc + n * 32 * 4);
    };
    auto load_frags = [&](const uint8_t* st, int sub) {
      const int alo = a_row0 + coff[sub][0], ahi = a_row0 + coff[sub][1];
      const int blo = b_row0 + coff[sub][0], bhi = b_row0 + coff[sub][1];
#pragma unroll
      for (int n = 0; n < FN; ++n) fb[n] = frag(st, blo + n * 32 * BK, bhi + n * 32 * BK);
#pragma unroll
      for (int m = 0; m < LIVE; ++m) fa[m] = frag(st, alo + m * 32 * BK, ahi + m * 32 * BK);
    };
    auto mma = [&](int sub) {
      const int sh = 8 * (2 * sub + lg);  // this lane's MX block of the step
#pragma unroll
      for (int m = 0; m < LIVE; ++m)
#pragma unroll
        for (int n = 0; n < FN; ++n)
          acc[m][n] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
              fa[m], fb[n], acc[m][n], 0, 0, 0, (int)(sa[m] >> sh), 0, (int)(sb[n] >> sh));
    };
#pragma unroll
    for (int s = 0; s < ST; ++s)
      if (s < nk) issue_any(stage_ptr(s), s, nt_c, live_c);
    if (ST - 1 < nk) __builtin_amdgcn_s_waitcnt(GLM_VMCNT(VPS * (ST - 1)));
    else __builtin_amdgcn_s_waitcnt(GLM_VMCNT(0));
    lds_barrier();

    auto step = [&](auto sc, int kt) {
      constexpr int s = decltype(sc)::value;
      uint8_t* cur = stage_ptr(s);
      if constexpr (LIVE > 0) load_scales(cur);
#pragma unroll
      for (int sub = 0; sub < KSUB; ++sub) {
        if constexpr (LIVE > 0) load_frags(cur, sub);
        if (sub == KSUB - 1 && kt + 1 < nk) {
          // all reads of this stage are issued: wait for stage kt+1, meet the
          // barrier (which also waits for this wave's reads), refill this stage
          if (kt + ST - 1 < nk) __builtin_amdgcn_s_waitcnt(GLM_VMCNT(VPS * (ST - 2)));
          else __builtin_amdgcn_s_waitcnt(GLM_VMCNT(0));
          lds_barrier();
          if (kt + ST < nk) issue_any(cur, kt + ST, nt_c, live_c);
        }
        if constexpr (LIVE > 0) mma(sub);
        // keep the next sub-step's fragment reads behind these MFMAs: one
        // sub-step of fragments in registers at a time
        __builtin_amdgcn_sched_barrier(0);
      }
    };
    for (int kt = 0; kt < nk; kt += ST) {
      unroll<ST>([&](auto uc) {
        constexpr int u = decltype(uc)::value;
        if (u == 0 || kt + u < nk) step(std::integral_constant<int, u>{}, kt + u);
      });
    }
  };
  // the main loop, specialised on the live row blocks and the copy hint
  auto go = [&](auto nt_c) {
    switch (live_m) {
      case 1: run(std::integral_constant<int, 1>{}, nt_c); break;
      case 2: if constexpr (FM >= 2) run(std::integral_constant<int, 2>{}, nt_c); break;
      case 3: if constexpr (FM >= 3) run(std::integral_constant<int, 3>{}, nt_c); break;
      case 4: if constexpr (FM >= 4) run(std::integral_constant<int, 4>{}, nt_c); break;
      default: run(std::integral_constant<int, 0>{}, nt_c); break;  // DMA and barriers only
    }
  };
  if constexpr (kStreamB<BM, BN>) {
    if (sole) go(std::true_type{});
    else go(std::false_type{});
  } else {
    go(std::false_type{});
  }

  // ------------------------------------------------------------ epilogue
  // accumulator element r of block (m, n): row 8*(r/4) + 4*(lane/32) + r%4,
  // column lane % 32
  auto row_of = [&](int m, int r) { return wrow0 + m * 32 + 8 * (r / 4) + 4 * lg + (r % 4); };
  if constexpr (MODE == GATE_UP) {
    const bool shared = (g == gu.E);
    const int F = shared ? gu.Fs : gu.F;
    const size_t hrow0 = (size_t)row0;
    uint8_t* Hq = (shared ? gu.Hs : gu.H) + hrow0 * F;
    // K-step-major scales over all rows of H (T * k) or Hs (T)
    const size_t hrows = shared ? (size_t)gu.T : (size_t)gu.T * gu.k;
    uint8_t* Hsc = (shared ? gu.Hssc : gu.Hsc) + hrow0 * 4;
#pragma unroll
    for (int m = 0; m < FM; ++m) {
      if (m >= live_m) continue;  // uniform across the wave
#pragma unroll
      for (int q = 0; q < FN / 2; ++q) {
        const int hblk = col0 / 32 + wn * TN / 64 + q;  // MX block of 32 hidden units
        const int hcol = hblk * 32 + lr;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const float h = silu(acc[m][2 * q][r]) * acc[m][2 * q + 1][r];
          // block maximum over the 32 lanes of this lane group (one row)
          float a = fabsf(h);
#pragma unroll
          for (int off = 16; off >= 1; off >>= 1) a = fmaxf(a, __shfl_xor(a, off, 32));
          const int s = mx_exponent(a);
          const uint32_t code = e4m3_code(ldexpf(h, -s));
          const int row = row_of(m, r);
          if (row < rows) {
            Hq[(size_t)row * F + hcol] = (uint8_t)code;
            if (lr == 0) Hsc[((size_t)(hblk / 4) * hrows + row) * 4 + hblk % 4] = (uint8_t)(s + 127);
          }
        }
      }
    }
  } else {
    // One 16-row half of a 32-row block at a time through this wave's slice
    // of stage 0, leaving as 16-byte pieces of four consecutive columns.
    constexpr int CG = TN / 4, RPP = kWave / CG;
    static_assert(kWave % CG == 0 && 16 % RPP == 0 && NW * 16 * TN * 4 <= C::STAGE,
                  "epilogue shape");
    float* blk = reinterpret_cast<float*>(lds0) + wave * (16 * TN);
    // row of Y and routing weight of every row of the tile
    if (tid < rows) {
      s_asg[tid] = g == dn.E ? (row0 + tid) * (dn.k + 1) + dn.k : y_row(row_a, dn.k);
      s_wt[tid] = row_wt;
    }
    __syncthreads();  // the row table is complete and every wave is done reading the stages
#pragma unroll
    for (int m = 0; m < FM; ++m) {
      if (m >= live_m) continue;
#pragma unroll
      for (int half = 0; half < 2; ++half) {
        // r in [8 half, 8 half + 8) covers rows [16 half, 16 half + 16) of the block
#pragma unroll
        for (int r = 8 * half; r < 8 * half + 8; ++r) {
          const int rb = row_of(m, r) - (wrow0 + m * 32 + 16 * half);
#pragma unroll
          for (int n = 0; n < FN; ++n) blk[rb * TN + n * 32 + lr] = acc[m][n][r];
        }
#pragma unroll
        for (int pass = 0; pass < 16 / RPP; ++pass) {
          const int rb = pass * RPP + lane / CG, cg = lane % CG;
          const int row = wrow0 + m * 32 + 16 * half + rb;
          const float4 v = *reinterpret_cast<const float4*>(blk + rb * TN + 4 * cg);
          if (row < rows) {
            const float w = s_wt[row];
            float* y = dn.Y + (size_t)s_asg[row] * dn.D + col0 + wn * TN + 4 * cg;
            store_stream(y, f32x4{w * v.x, w * v.y, w * v.z, w * v.w});
          }
        }
      }
    }
  }
}

// One thread per 32-element block of x: block maximum, scale, codes.  The
// scale goes to the K-step-major array [D/128][T][4].
__global__ __launch_bounds__(256) void quantize_mx_kernel(const bf16_t* __restrict__ x,
                                                          uint8_t* __restrict__ xq,
                                                          uint8_t* __restrict__ xs, int T,
                                                          int nb) {
  const size_t b = (size_t)blockIdx.x * 256 + threadIdx.x;
  if (b >= (size_t)T * nb) return;
  const uint4* p = reinterpret_cast<const uint4*>(x + b * 32);
  uint32_t u[16];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint4 v = p[i];
    u[4 * i] = v.x; u[4 * i + 1] = v.y; u[4 * i + 2] = v.z; u[4 * i + 3] = v.w;
  }
  float a = 0.f;
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    a = fmaxf(a, fabsf(__uint_as_float(u[i] << 16)));
    a = fmaxf(a, fabsf(__uint_as_float(u[i] & 0xFFFF0000u)));
  }
  const int s = mx_exponent(a);
  uint32_t c[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const uint32_t c0 = e4m3_code(ldexpf(__uint_as_float(u[2 * i] << 16), -s));
    const uint32_t c1 = e4m3_code(ldexpf(__uint_as_float(u[2 * i] & 0xFFFF0000u), -s));
    const uint32_t c2 = e4m3_code(ldexpf(__uint_as_float(u[2 * i + 1] << 16), -s));
    const uint32_t c3 = e4m3_code(ldexpf(__uint_as_float(u[2 * i + 1] & 0xFFFF0000u), -s));
    c[i] = c0 | (c1 << 8) | (c2 << 16) | (c3 << 24);
  }
  uint4* q = reinterpret_cast<uint4*>(xq + b * 32);
  q[0] = make_uint4(c[0], c[1], c[2], c[3]);
  q[1] = make_uint4(c[4], c[5], c[6], c[7]);
  const int t = (int)(b / nb), j = (int)(b % nb);
  xs[((size_t)(j / 4) * T + t) * 4 + j % 4] = (uint8_t)(s + 127);
}

// Input scales into expert-row order, one thread per output dword.
__global__ __launch_bounds__(256) void permute_scales_kernel(const uint32_t* __restrict__ xs,
                                                             const int32_t* __restrict__ row_assign,
                                                             int T, int k, size_t rows, size_t n_dw,
                                                             uint32_t* __restrict__ xsp) {
  const size_t i = (size_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= n_dw) return;
  const size_t kt = i / rows, r = i % rows;
  xsp[i] = xs[kt * T + row_assign[r] / k];
}

// Row-major scales [n_mats][N][K/32] -> K-step-major [n_mats][K/128][N][4]:
// one thread per output dword (four consecutive scales of one row).
__global__ __launch_bounds__(256) void pack_scales_kernel(const uint8_t* __restrict__ src,
                                                          uint8_t* __restrict__ dst,
                                                          size_t n_dw, int N, int ksteps) {
  const size_t i = (size_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= n_dw) return;
  const size_t per = (size_t)N * ksteps;  // dwords per matrix
  const size_t m = i / per;
  const int r = (int)(i % per);
  const int kt = r / N, n = r % N;
  const uint32_t v = *reinterpret_cast<const uint32_t*>(src + (m * N + n) * (size_t)ksteps * 4 +
                                                        (size_t)kt * 4);
  reinterpret_cast<uint32_t*>(dst)[i] = v;
}

// Tile configurations <BM, BN, WM, WN, stages>.  The prefill tile is
// 256 x 128: at one byte per element it moves fewer bytes per flop than the
// bf16 256 x 256 tile, and its 64 accumulator registers per wave leave room
// for a third stage.
// The decode tile keeps two stages (76 KB of LDS), so two workgroups share a
// CU and one's tile setup and first copies overlap the other's weight stream.
#ifndef GLM_MX_CFG_BIG
#define GLM_MX_CFG_BIG 256, 128, 4, 2, 3
#endif
#ifndef GLM_MX_CFG_DECODE
#define GLM_MX_CFG_DECODE 32, 256, 1, 4, 2
#endif
using MxDecode = Cfg<GLM_MX_CFG_DECODE>;
#ifndef GLM_MX_CFG_MID
#define GLM_MX_CFG_MID 128, 256, 2, 4, 3
#endif
using MxMid = Cfg<GLM_MX_CFG_MID>;
using MxBig = Cfg<GLM_MX_CFG_BIG>;
using MxNarrow = Cfg<32, 64, 1, 1, 4>;

template <class C, int MODE>
hipError_t launch_one(const MxGateUpArgs& gu, const MxDownArgs& dn, unsigned grid,
                      hipStream_t s) {
  if (grid == 0) return hipSuccess;
  grouped_gemm_mx_kernel<C, MODE><<<grid, C::NT, 0, s>>>(gu, dn);
  return hipGetLastError();
}

template <int MODE>
hipError_t dispatch(GemmShape sh, const MxGateUpArgs& gu, const MxDownArgs& dn, unsigned grid,
                    hipStream_t s) {
  if (sh.BM == MxDecode::BM && sh.BN == MxDecode::BN)
    return launch_one<MxDecode, MODE>(gu, dn, grid, s);
  if (sh.BM == MxMid::BM && sh.BN == MxMid::BN) return launch_one<MxMid, MODE>(gu, dn, grid, s);
  if (sh.BM == MxBig::BM && sh.BN == MxBig::BN) return launch_one<MxBig, MODE>(gu, dn, grid, s);
  if (sh.BM == MxNarrow::BM && sh.BN == MxNarrow::BN)
    return launch_one<MxNarrow, MODE>(gu, dn, grid, s);
  return hipErrorInvalidValue;
}

}  // namespace gemm_mx

GemmShape gemm_shape_mx(double rows_per_group, bool wide) {
  using namespace gemm_mx;
  if (!wide) return {MxNarrow::BM, MxNarrow::BN};
  if (rows_per_group <= 24.0) return {MxDecode::BM, MxDecode::BN};
#ifndef GLM_MX_MID_MAX_ROWS
#define GLM_MX_MID_MAX_ROWS 96.0
#endif
  if (rows_per_group <= GLM_MX_MID_MAX_ROWS) return {MxMid::BM, MxMid::BN};
  return {MxBig::BM, MxBig::BN};
}

hipError_t launch_quantize_mx(const bf16_t* x, uint8_t* xq, uint8_t* xs, int T, int D,
                              hipStream_t s) {
  const size_t nblk = (size_t)T * (D / 32);
  if (nblk == 0) return hipSuccess;
  gemm_mx::quantize_mx_kernel<<<(unsigned)((nblk + 255) / 256), 256, 0, s>>>(x, xq, xs, T,
                                                                             D / 32);
  return hipGetLastError();
}

hipError_t launch_permute_mx_scales(const uint8_t* xs, const int32_t* row_assign, int T, int k,
                                    int D, uint8_t* xsp, hipStream_t s) {
  const size_t rows = (size_t)T * k, n_dw = rows * (D / 128);
  if (n_dw == 0) return hipSuccess;
  gemm_mx::permute_scales_kernel<<<(unsigned)((n_dw + 255) / 256), 256, 0, s>>>(
      reinterpret_cast<const uint32_t*>(xs), row_assign, T, k, rows, n_dw,
      reinterpret_cast<uint32_t*>(xsp));
  return hipGetLastError();
}

hipError_t launch_pack_mx_scales(const uint8_t* src, uint8_t* dst, size_t n_mats, int N, int K,
                                 hipStream_t s) {
  const size_t n_dw = n_mats * (size_t)N * (K / 128);
  if (n_dw == 0) return hipSuccess;
  gemm_mx::pack_scales_kernel<<<(unsigned)((n_dw + 255) / 256), 256, 0, s>>>(src, dst, n_dw, N,
                                                                             K / 128);
  return hipGetLastError();
}

hipError_t launch_gateup_mx(const MxGateUpArgs& a, GemmShape sh, hipStream_t s) {
  return gemm_mx::dispatch<gemm_mx::GATE_UP>(sh, a, MxDownArgs{}, (unsigned)a.grid, s);
}

hipError_t launch_down_mx(const MxDownArgs& a, GemmShape sh, hipStream_t s) {
  return gemm_mx::dispatch<gemm_mx::DOWN>(sh, MxGateUpArgs{}, a, (unsigned)a.grid, s);
}

}  // namespace glm
