// Internal declarations shared by the HIP kernels and the C-ABI host code of
// the GLM-5.2 MoE layer (gfx950 only).
#pragma once

#include <hip/hip_runtime.h>

#include <type_traits>
#include <utility>
#include <stdint.h>
#include <stddef.h>

namespace glm {

// ------------------------------------------------------------ vector types
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint16_t bf16_t;  // bf16 bit pattern in memory

constexpr int kWave = 64;
constexpr int kMaxExperts = 256;
constexpr int kMaxTopK = 32;
constexpr int kTokTile = 64;   // tokens per routing tile (one bit per token in a u64 mask)
constexpr int kXcds = 8;       // MI355X: 8 XCDs, workgroups dispatched round-robin over them
// Consecutive logical tiles kept on one XCD (see xcd_tile): kXcdBlock in
// general; on 256-row tiles, kXcdBlockRoutedGu for the bf16 gate/up GEMM of
// routed experts and kXcdBlockMxGu / kXcdBlockMxDn for the MXFP8 GEMMs; on
// 32-row (decode) tiles kXcdBlockDecodeDn for the bf16 down GEMM (measured
// per launch kind).
#ifndef GLM_XCD_BLOCK
#define GLM_XCD_BLOCK 64
#endif
#ifndef GLM_XCD_BLOCK_ROUTED_GU
#define GLM_XCD_BLOCK_ROUTED_GU 16
#endif
#ifndef GLM_XCD_BLOCK_MX_GU
#define GLM_XCD_BLOCK_MX_GU 32
#endif
#ifndef GLM_XCD_BLOCK_MX_DN
#define GLM_XCD_BLOCK_MX_DN 128
#endif
constexpr int kXcdBlock = GLM_XCD_BLOCK, kXcdBlockRoutedGu = GLM_XCD_BLOCK_ROUTED_GU;
constexpr int kXcdBlockMxGu = GLM_XCD_BLOCK_MX_GU, kXcdBlockMxDn = GLM_XCD_BLOCK_MX_DN;
#ifndef GLM_XCD_BLOCK_DECODE_DN
#define GLM_XCD_BLOCK_DECODE_DN 128
#endif
constexpr int kXcdBlockDecodeDn = GLM_XCD_BLOCK_DECODE_DN;
#ifndef GLM_XCD_BLOCK_FEW  // the dense layer's few decode tiles (both GEMMs)
#define GLM_XCD_BLOCK_FEW 1
#endif
// Average rows per expert up to which the two-stage gate/up and down GEMMs
// issue each refill before their wait (GateUpArgs::early, DownArgs::early).
// Measured: the two orders are equal at 160 rows per expert, the plain order
// is faster at 192.
#ifndef GLM_EARLY_MAX_ROWS
#define GLM_EARLY_MAX_ROWS 160.0
#endif
#ifndef GLM_ZIP  // rounds of the longest-first lists zipped (zip_position):
#define GLM_ZIP 3  // bit 0 gate/up list, bit 1 down list
#endif

// Cache policy of the weight-row copies.  The only row tile of a group is the
// only reader of the group's weight rows in a launch, so on decode tiles (at
// most GLM_STREAM_B_MAX_BM rows, at least 128 columns) those rows are copied
// with the non-temporal hint and do not displace reused lines; groups with
// several row tiles share each weight row through L2.  The narrow 64-column
// tiles (dense layers on decode batches) keep plain copies.
#ifndef GLM_STREAM_B_MAX_BM
#define GLM_STREAM_B_MAX_BM 128
#endif
constexpr int32_t kSoleRowTile = 1 << 16;  // TileDesc::group flag
constexpr int32_t kGroupMask = kSoleRowTile - 1;
constexpr int32_t kChunkTile = 1 << 17;  // TileDesc::group flag: a gate/up K chunk
// TileDesc::group bits 20 and up: K chunk of a tile of the shared (dense)
// group when its contraction is split (DownArgs::ksplit > 1; gate/up tiles
// flagged kChunkTile)
constexpr int kKChunkShift = 20;
constexpr int kCpolNt = 2;  // cache-policy immediate of the LDS-DMA load: NT
template <int BM, int BN>
constexpr bool kStreamB = BM <= GLM_STREAM_B_MAX_BM && BN >= 128;

// Store of a slot row piece that is read once, by the combine pass: a
// non-temporal store, so the 4-byte-per-element slot rows do not displace
// the weight and activation lines the grouped GEMMs are still reading from L2.
__device__ __forceinline__ void store_stream(float* p, f32x4 v) {
  __builtin_nontemporal_store(v, reinterpret_cast<f32x4*>(p));
}
__device__ __forceinline__ void store_stream(float* p, float v) { __builtin_nontemporal_store(v, p); }

// Work item of a grouped GEMM launch: one BM x BN output tile of one group.
struct TileDesc {
  int32_t group;   // expert id (E: the shared expert), | kSoleRowTile when the group has
                   // one row tile, i.e. this tile is the only reader of the group's weights
  int32_t row0;    // first row of the tile: routed groups count in the expert-sorted
                   // rows (the group's offset included), the shared expert in tokens
  int32_t rows;    // valid rows in the tile (1..BM)
  int32_t col0;    // first output column (gate/up: first hidden column)
};

// Tile shapes chosen by the host for one grouped GEMM launch.
struct GemmShape {
  int BM, BN;
};

// ------------------------------------------------------- launch wrappers
// Each returns hipGetLastError() after enqueueing on `s`.

// Token rows per router-logits workgroup for a batch of T tokens.
int router_tile_rows(int T);
// Router logits.  partial[ks][T][E] fp32 = x[:, kslice] . router_w[:, kslice]^T.
// Both also clear masks[ceil(T/64)][E] for the top-k kernel.
hipError_t launch_router_logits_bf16(const bf16_t* x, const float* router_w, float* partial,
                                     int T, int D, int E, int ksplit, int kchunk,
                                     uint64_t* masks, hipStream_t s);
hipError_t launch_router_logits_f32(const float* x, const float* router_w, float* partial,
                                    int T, int D, int E, uint64_t* masks, hipStream_t s);

// Sum partials, sigmoid, biased top-k, renormalise and scale; per-64-token
// tile expert membership masks.
// Group-limited selection when n_group > 1 (keep the topk_group groups with
// the largest sum of their group_topk best biased scores).
struct GroupRouting {
  int n_group, topk_group, group_topk;
};
hipError_t launch_router_topk(const float* partial, int ksplit, const float* corr_bias,
                              int T, int E, int k, float scale, GroupRouting gr,
                              int32_t* topk_idx, float* topk_w, uint64_t* masks,
                              hipStream_t s);

// Per-expert counts and offsets, per-(tile, expert) row bases, and the tile
// lists of the two grouped GEMMs.
struct ScanParams {
  int T, E, k, F, Fs, D;
  GemmShape gu, dn;
  int gu_desc_cap, dn_desc_cap;
  int dn_ksplit;               // K chunks of the shared group's down tiles (1: whole K)
  // the shared group's gate/up tiles: the first gu_whole in column-tile-major
  // order run whole, the others in gu_ksplit K chunks each; gu_shared_n is
  // the number of descriptors (whole tiles plus chunks)
  int gu_ksplit, gu_whole, gu_shared_n;
  // XCD block (xcd_tile) of each launch whose longest-first list is zipped
  // round by round (zip_position), 0: listing order
  int gu_zip, dn_zip;
};
hipError_t launch_scan(const uint64_t* masks, const ScanParams& p,
                       int32_t* counts, int32_t* offsets, int32_t* tile_base,
                       TileDesc* gu_desc, int32_t* gu_count,
                       TileDesc* dn_desc, int32_t* dn_count, hipStream_t s);

// Stable expert-major permutation: row_assign[row] = t * k + j, and the
// routing weight of that row, row_w[row] = topk_w[t * k + j].
hipError_t launch_scatter(const int32_t* topk_idx, const uint64_t* masks,
                          const int32_t* tile_base, const float* topk_w, int T, int E, int k,
                          int32_t* row_assign, float* row_w, hipStream_t s);

// bf16 grouped GEMMs.
struct GateUpArgs {
  const bf16_t* x;             // [T][D]
  const int32_t* row_assign;   // [T*k]
  const bf16_t* w1;            // [E][F][D]
  const bf16_t* w3;
  const bf16_t* sw1;           // [Fs][D]
  const bf16_t* sw3;
  const TileDesc* desc;
  const int32_t* desc_count;
  bf16_t* H;                   // [T*k][F]
  bf16_t* Hs;                  // [T][Fs]
  int T, D, E, F, Fs, k;
  int grid;                    // launched workgroups (>= desc_count, multiple of 8)
  int xblk;                    // XCD block of the tile mapping (xcd_tile)
  int early;                   // two-stage tiles: issue each refill before the wait
  // K chunks of the shared group's tiles flagged kChunkTile (a dense layer on
  // a decode-size batch only): chunk kc of such a tile writes its fp32 sums
  // for hidden column pc0 + c, gate to P[kc][t][c] and up to P[kc][t][pw + c],
  // and launch_gateup_fixup forms those columns of Hs
  int ksplit;
  float* P;
  int pc0, pw;
};
// Tile shape of a grouped GEMM launch.  `wide` says the output width allows
// the 256-column tiles (gate/up: F and F_shared multiples of 128; down and
// shared-combine: D a multiple of 256); otherwise 64-column tiles are used.
GemmShape gemm_shape(double rows_per_group, bool wide);
// Tile shape for a single group of `rows` (at most 96) rows: the dense layer
// on a decode-size batch.
GemmShape gemm_shape_few(int rows, bool wide);
// Workgroups of a bf16 tile shape's kernel that fit on one CU at once.
int gemm_wgs_per_cu(GemmShape sh);

hipError_t launch_gateup_bf16(const GateUpArgs& a, GemmShape sh, hipStream_t s);
// Hs[t][c0 + c] = bf16(SiLU(sum_kc P[kc][t][c]) * sum_kc P[kc][t][w + c]) for
// c < w, chunks summed in order (c0 and w multiples of 4).
hipError_t launch_gateup_fixup(const float* P, bf16_t* Hs, int T, int Fs, int c0, int w, int ks,
                               hipStream_t s);

struct DownArgs {
  const bf16_t* H;             // [T*k][F]
  const bf16_t* Hs;            // [T][Fs]
  const int32_t* row_assign;
  const bf16_t* w2;            // [E][D][F]
  const bf16_t* sw2;           // [D][Fs]
  const float* row_w;          // [T*k] routing weight of each expert-sorted row
  const TileDesc* desc;        // tiles of the routed groups and the shared expert (group E)
  const int32_t* desc_count;
  float* Y;                    // [T][k+ksplit][D]: slot j < k routed (weighted), slots
                               // k .. k+ksplit-1 the shared group's K chunks
  int T, D, E, F, Fs, k;
  int ksplit;                  // K chunks of the shared group (only without routed groups)
  int grid;
  int xblk;
  int early;                   // two-stage tiles: issue each refill before the wait
};
hipError_t launch_down_bf16(const DownArgs& a, GemmShape sh, hipStream_t s);

// out[t] = Y[t][k] + sum_{j<k} Y[t][j] (+ residual[t]): the shared expert's
// output, then the weighted routed outputs in slot order, then the residual
// stream when `residual` is non-null (bf16 or fp32 per res_bf16).
hipError_t launch_combine(const float* Y, float* out, int T, int D, int k, const void* residual,
                          bool res_bf16, hipStream_t s);

// MXFP8 grouped GEMMs (OCP MX: E4M3 codes, one E8M0 scale per 32 elements
// along the contraction dimension; scale arrays are [rows][K/32] bytes).
struct MxGateUpArgs {
  const uint8_t* xq;           // [T][D]   layer input, quantised per token
  const uint8_t* xs;           // [D/128][T][4] (scales K-step-major)
  const uint8_t* xsp;          // [D/128][T*k][4]: the same scales in expert-row order
  const int32_t* row_assign;
  const uint8_t* w1; const uint8_t* w1s;   // [E][F][D], [E][D/128][F][4]
  const uint8_t* w3; const uint8_t* w3s;
  const uint8_t* sw1; const uint8_t* sw1s; // [Fs][D], [D/128][Fs][4]
  const uint8_t* sw3; const uint8_t* sw3s;
  const TileDesc* desc;
  const int32_t* desc_count;
  uint8_t* H; uint8_t* Hsc;    // [T*k][F], [F/128][T*k][4]: gated hidden rows, quantised
  uint8_t* Hs; uint8_t* Hssc;  // [T][Fs], [Fs/128][T][4]
  int T, D, E, F, Fs, k;
  int grid;
  int xblk;
};
struct MxDownArgs {
  const uint8_t* H; const uint8_t* Hsc;
  const uint8_t* Hs; const uint8_t* Hssc;
  const int32_t* row_assign;
  const uint8_t* w2; const uint8_t* w2s;   // [E][D][F], [E][F/128][D][4]
  const uint8_t* sw2; const uint8_t* sw2s; // [D][Fs], [Fs/128][D][4]
  const float* row_w;
  const TileDesc* desc;
  const int32_t* desc_count;
  float* Y;                    // as DownArgs
  int T, D, E, F, Fs, k;
  int grid;
  int xblk;
};
// x (bf16 [T][D]) -> MXFP8 codes [T][D] and K-step-major scales [D/128][T][4].
hipError_t launch_quantize_mx(const bf16_t* x, uint8_t* xq, uint8_t* xs, int T, int D,
                              hipStream_t s);
// Input scales in expert-row order: xsp[kt][row] = xs[kt][row_assign[row] / k]
// (dwords), so a tile's routed rows read contiguous scales.
hipError_t launch_permute_mx_scales(const uint8_t* xs, const int32_t* row_assign, int T, int k,
                                    int D, uint8_t* xsp, hipStream_t s);
// Row-major MX scales [n_mats][N][K/32] -> K-step-major [n_mats][K/128][N][4].
hipError_t launch_pack_mx_scales(const uint8_t* src, uint8_t* dst, size_t n_mats, int N, int K,
                                 hipStream_t s);
// Tile shape of an MXFP8 grouped GEMM launch (same `wide` rule as gemm_shape).
GemmShape gemm_shape_mx(double rows_per_group, bool wide);
hipError_t launch_gateup_mx(const MxGateUpArgs& a, GemmShape sh, hipStream_t s);
hipError_t launch_down_mx(const MxDownArgs& a, GemmShape sh, hipStream_t s);

// Pre-norm block: out = h / sqrt(mean(h^2) + eps) * w per row, computed in
// fp64 and rounded once to the activation dtype (bf16 or fp32).
hipError_t launch_rmsnorm(const void* h, const float* w, void* out, int T, int D, float eps,
                          bool bf16, hipStream_t s);

// fp32 path (plain kernels; same data flow).
struct F32Args {
  const float* x;
  const int32_t* row_assign;
  const int32_t* offsets;
  const float* w1; const float* w3; const float* w2;
  const float* sw1; const float* sw3; const float* sw2;
  const float* topk_w;
  float* H; float* Hs; float* Y; float* out;
  const float* residual;       // nullable: added to out last
  int T, D, E, F, Fs, k;
};
hipError_t launch_gateup_f32(const F32Args& a, hipStream_t s);
hipError_t launch_down_f32(const F32Args& a, hipStream_t s);
hipError_t launch_shared_combine_f32(const F32Args& a, hipStream_t s);

// Row of Y holding assignment a = t * k + j (slot j of token t).
__host__ __device__ inline int y_row(int a, int k) { return (a / k) * (k + 1) + a % k; }

// ------------------------------------------------------------- helpers

typedef __attribute__((address_space(3))) void lds_void;

// s_waitcnt immediate: vector-memory count N, other counters left alone.
#define GLM_VMCNT(N) (((N) & 0xF) | (((N) >> 4) << 14) | (7 << 4) | (0xF << 8))

// f(integral_constant<int, 0>), ..., f(integral_constant<int, N-1>), in order.
template <int... I, class F>
__device__ __forceinline__ void unroll_impl(std::integer_sequence<int, I...>, F&& f) {
  (f(std::integral_constant<int, I>{}), ...);
}
template <int N, class F>
__device__ __forceinline__ void unroll(F&& f) {
  unroll_impl(std::make_integer_sequence<int, N>{}, f);
}

// Workgroup barrier after this wave's LDS operations have completed (and
// nothing else: outstanding global loads stay in flight).
__device__ __forceinline__ void lds_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

__host__ __device__ inline int cdiv(int a, int b) { return (a + b - 1) / b; }

// Physical place of logical position i of a list of n tiles listed longest
// first and cut into units of `unit` tiles (the last, partial unit keeps its
// place): of the nb full units, logical unit b goes to unit 2b when
// b < ceil(nb / 2) and to unit 2 (nb - 1 - b) + 1 otherwise, so the heaviest
// and the lightest units alternate.  A permutation of [0, n).
__host__ __device__ inline int zip_position(int i, int n, int unit) {
  if (unit <= 0) return i;
  const int nb = n / unit, b = i / unit;
  if (b >= nb) return i;
  const int half = (nb + 1) / 2;
  const int pb = b < half ? 2 * b : 2 * (nb - 1 - b) + 1;
  return pb * unit + i % unit;
}
// One dispatch round of xcd_tile over a list of n tiles with XCD block xb:
// a block of consecutive tiles for each XCD (0: no zipping).
__host__ __device__ inline int xcd_round(int n, int xb) {
  if (n <= 0 || xb <= 0) return 0;
  const int rounds = cdiv(n, kXcds * xb);
  return kXcds * cdiv(n, kXcds * rounds);
}

// Workgroup -> logical tile of a grouped GEMM launch.  Workgroups are
// dispatched round-robin over the XCDs (workgroup b on XCD b % 8).  The n
// tiles of the list are cut into 8R blocks of about n / 8R consecutive tiles
// (R = ceil(n / (8 xb)) rounds), dealt to the XCDs in turn, and each
// XCD walks its R blocks in order.  Tiles sharing an expert's gathered rows
// or weight slice (neighbours in the list) run on one XCD and its L2, every
// XCD gets the same number of tiles up to one, and a run of expensive tiles
// (a hot expert's) spreads over all XCDs.  Returns -1 past the list.
__device__ inline int xcd_tile(int n, int xb) {
  if (n <= 0) return -1;
  const int x = blockIdx.x % kXcds, o = blockIdx.x / kXcds;
  const int rounds = cdiv(n, kXcds * xb);
  const int blk = cdiv(n, kXcds * rounds);  // 1 .. xb
  const int r = o / blk;
  if (r >= rounds) return -1;
  const int i = (x + kXcds * r) * blk + o % blk;
  return i < n ? i : -1;
}
// Launch width covering every tile of a list of at most cap tiles
// (each XCD walks at most xb * ceil(cap / 8 xb) ordinals).
inline int xcd_grid(int cap, int xb) {
  return kXcds * xb * cdiv(cdiv(cap, xb), kXcds);
}

__device__ inline float bf16_to_f32(bf16_t v) {
  return __uint_as_float(static_cast<uint32_t>(v) << 16);
}

// fp32 -> bf16, round to nearest even (finite inputs).
__device__ inline bf16_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return static_cast<bf16_t>(u >> 16);
}

}  // namespace glm
