// C ABI of the GLM-5.2 MoE layer: argument checks, workspace plan and the
// launch sequence [rmsnorm ->] router -> top-k -> scan -> scatter -> gate/up
// -> down -> combine [+ residual], all on the caller's stream.  The dense
// feed-forward entry runs the same kernels with the shared group only.
#include "glm_moe.h"
#include "common.h"

#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <mutex>
#include <new>
#include <vector>

using namespace glm;

namespace {

thread_local char g_err[512] = "";

int fail(int code, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof g_err, fmt, ap);
  va_end(ap);
  return code;
}

constexpr size_t kAlign = 256;
size_t align_up(size_t v) { return (v + kAlign - 1) / kAlign * kAlign; }

// Workspace regions (byte offsets) and launch parameters of one call.
struct Plan {
  int T, D, E, F, Fs, k;
  bool bf16;         // bf16 activations
  bool mx;           // MXFP8 expert weights (H, Hs hold E4M3 codes)
  bool dense;        // no routed experts: the shared group only
  int ntiles;        // 64-token routing tiles
  int ksplit, kchunk;
  GemmShape gu, dn;
  int gu_cap, dn_cap;
  int dn_ksplit;     // K chunks of the shared (dense) group's down tiles
  int gu_ksplit;     // K chunks of its gate/up tiles past the first gu_whole
  int gu_whole, gu_shared_n;  // (see ScanParams)
  int gu_pc0, gu_pw;          // hidden columns [pc0, pc0 + pw) come from K chunks
  bool few_tiles;             // dense layer on a decode-size batch
  GroupRouting gr;
  const float* norm_weight;
  float norm_eps;
  bool add_residual;
  size_t xnorm, partial, idx, w, masks, tile_base, counts, offsets, gu_count, dn_count, gu_desc,
      dn_desc, row_assign, row_w, H, Hs, Y, Pgu, xq, xs, xsp, Hsc, Hssc;
  size_t total;
};

// K chunks for the few tiles of a dense layer on a decode-size batch: the
// divisor ks of the K steps, in chunks of at least 16 steps, that minimises
// the rounds of tiles * ks over the 256 CUs (`per_cu` workgroups each) times
// (steps per chunk + 4), the last term a tile's fixed cost (pipeline fill,
// epilogue) counted in K steps.
int ksplit_for(int tiles, int ksteps, int per_cu) {
  const int slots = 256 * (per_cu > 0 ? per_cu : 1);
  int best = 1;
  long long best_t = -1;
  for (int ks = 1; ks == 1 || ks <= ksteps / 16; ++ks) {
    if (ksteps % ks) continue;
    const long long t = (long long)cdiv(tiles * ks, slots) * (ksteps / ks + 4);
    if (best_t < 0 || t < best_t) { best_t = t; best = ks; }
  }
  return best;
}

// Gate/up K split of the dense layer on a decode-size batch.  With `slots`
// = 256 CUs x `per_cu` workgroups and the tiles listed column-tile major
// (`mt` row tiles per column): the last tiles % slots tiles, rounded up to
// whole columns, run in *ks K chunks and the others (*whole) run whole, ks
// the largest divisor of the K steps with (tiles - *whole) * ks <= slots and
// chunks of at least 8 steps, so every slot gets at most one chunk and every
// CU streams about the same number of K steps.  With fewer tiles than slots
// every tile runs in chunks (ksplit_for); without a remainder none does.
void plan_gateup_split(int tiles, int mt, int ksteps, int per_cu, int* whole, int* ks) {
  const int slots = 256 * (per_cu > 0 ? per_cu : 1);
  *whole = tiles;
  *ks = 1;
  if (tiles <= 0 || mt <= 0) return;
  if (tiles < slots) {
    *ks = ksplit_for(tiles, ksteps, per_cu);
    *whole = *ks > 1 ? 0 : tiles;
    return;
  }
  int rest = tiles % slots;
  rest = cdiv(rest, mt) * mt;
  if (rest == 0) return;
  int best = 1;
  for (int c = 2; c * 8 <= ksteps; ++c)
    if (ksteps % c == 0 && (long long)rest * c <= slots) best = c;
  if (best < 2) return;
  *whole = tiles - rest;
  *ks = best;
}

int desc_cap(int A, int E, GemmShape s, int ncol_tiles) {
  const long nz = A < E ? A : E;
  const long mt = ((long)A + (long)(s.BM - 1) * nz) / s.BM;
  return (int)(mt * ncol_tiles);
}

int check_options(const glm_moe_options* o, int E, int top_k, bool dense, Plan& P) {
  P.gr = GroupRouting{1, 1, 2};
  P.norm_weight = nullptr;
  P.norm_eps = 0.f;
  P.add_residual = false;
  if (!o) return GLM_MOE_OK;
  if (!dense && o->n_group > 1) {
    const int ng = o->n_group;
    if (ng > 64) return fail(GLM_MOE_EUNSUPPORTED, "n_group=%d > 64", ng);
    if (E % ng) return fail(GLM_MOE_EINVAL, "E=%d is not a multiple of n_group=%d", E, ng);
    const int gsz = E / ng;
    const int gk = o->group_topk == 0 ? (gsz < 2 ? gsz : 2) : o->group_topk;
    if (o->topk_group < 1 || o->topk_group > ng)
      return fail(GLM_MOE_EINVAL, "topk_group=%d outside [1, %d]", o->topk_group, ng);
    if (gk < 1 || gk > gsz)
      return fail(GLM_MOE_EINVAL, "group_topk=%d outside [1, %d]", gk, gsz);
    if (o->topk_group * gsz < top_k)
      return fail(GLM_MOE_EINVAL, "topk_group*E/n_group=%d < top_k=%d", o->topk_group * gsz,
                  top_k);
    P.gr = GroupRouting{ng, o->topk_group, gk};
  } else if (!dense && o->n_group < 0) {
    return fail(GLM_MOE_EINVAL, "n_group=%d < 0", o->n_group);
  }
  if (o->norm_weight) {
    if (!(o->norm_eps >= 0.f) || !std::isfinite(o->norm_eps))
      return fail(GLM_MOE_EINVAL, "norm_eps must be finite and >= 0");
    if (reinterpret_cast<uintptr_t>(o->norm_weight) & 15)
      return fail(GLM_MOE_EINVAL, "norm_weight is not 16-byte aligned");
    P.norm_weight = o->norm_weight;
    P.norm_eps = o->norm_eps;
  }
  P.add_residual = o->add_residual != 0;
  return GLM_MOE_OK;
}

int make_plan(const glm_moe_dims* d, int top_k, const glm_moe_options* opts, bool dense,
              Plan* p) {
  if (!d) return fail(GLM_MOE_EINVAL, "dims is null");
  if (d->T < 0 || d->D <= 0 || d->F_shared <= 0 || (!dense && (d->E <= 0 || d->F <= 0)))
    return fail(GLM_MOE_EINVAL, "bad sizes T=%d D=%d E=%d F=%d F_shared=%d", d->T, d->D, d->E,
                d->F, d->F_shared);
  if (!dense && d->E > kMaxExperts)
    return fail(GLM_MOE_EUNSUPPORTED, "E=%d exceeds %d experts", d->E, kMaxExperts);
  if (!dense) {
    const int kmax = d->E < kMaxTopK ? d->E : kMaxTopK;
    if (top_k < 1 || top_k > kmax)
      return fail(GLM_MOE_EINVAL, "top_k=%d outside [1, %d]", top_k, kmax);
  }
  const bool mx = d->act_dtype == GLM_MOE_BF16 && d->weight_dtype == GLM_MOE_MXFP8;
  if (!mx && (d->act_dtype != d->weight_dtype ||
              (d->act_dtype != GLM_MOE_F32 && d->act_dtype != GLM_MOE_BF16)))
    return fail(GLM_MOE_EUNSUPPORTED,
                "dtype pair act=%d weight=%d (supported: f32/f32, bf16/bf16, bf16/mxfp8)",
                d->act_dtype, d->weight_dtype);
  if (mx && dense)
    return fail(GLM_MOE_EUNSUPPORTED, "the dense FFN takes f32 or bf16 weights");
  const bool bf16 = d->act_dtype == GLM_MOE_BF16;
  if (bf16 && (d->D % 64 || d->F_shared % 64 || (!dense && d->F % 64)))
    return fail(GLM_MOE_EUNSUPPORTED, "bf16 path needs D, F, F_shared multiples of 64 (D=%d F=%d Fs=%d)",
                d->D, d->F, d->F_shared);
  if (mx && (d->D % 128 || d->F % 128 || d->F_shared % 128))
    return fail(GLM_MOE_EUNSUPPORTED, "MXFP8 path needs D, F, F_shared multiples of 128 (D=%d F=%d Fs=%d)",
                d->D, d->F, d->F_shared);
  if ((long long)d->T * (dense ? 1 : top_k) > (1ll << 30))
    return fail(GLM_MOE_EUNSUPPORTED, "T*top_k=%lld too large", (long long)d->T * top_k);

  Plan& P = *p;
  int st = check_options(opts, d->E, top_k, dense, P);
  if (st) return st;
  P.dense = dense;
  P.T = d->T; P.D = d->D; P.Fs = d->F_shared;
  P.E = dense ? 0 : d->E;
  P.F = dense ? 0 : d->F;
  P.k = dense ? 0 : top_k;
  P.bf16 = bf16;
  P.mx = mx;
  const int T = P.T, A = T * P.k;
  P.ntiles = cdiv(T, kTokTile);

  if (bf16) {
    // enough (token tile, expert group, K slice) workgroups to cover the chip
    const int base = cdiv(T, router_tile_rows(T)) * cdiv(P.E > 0 ? P.E : 1, 64);
    int ks = cdiv(512, base > 0 ? base : 1);
    const int ksteps = P.D / 64;
    if (ks > 24) ks = 24;
    if (ks > ksteps) ks = ksteps;
    if (ks < 1) ks = 1;
    P.kchunk = cdiv(ksteps, ks) * 64;
    P.ksplit = cdiv(P.D, P.kchunk);
    const double per_group = dense ? (double)T : (double)A / P.E;
    const bool wide_gu = (dense || P.F % 128 == 0) && P.Fs % 128 == 0;
    const bool wide_dn = P.D % 256 == 0;
    // A dense layer on a decode-size batch is a single group of a few rows:
    // its weights are streamed on the decode tiles (32 or 64 x 128, one row
    // tile up to 64 tokens), and both GEMMs, whose few column tiles would
    // leave CUs idle or fill them unevenly (288 gate/up and 48 down tiles at
    // 64 tokens, hidden 6144, width 18432), split their contraction into K
    // chunks: down chunks write separate slots of Y, summed in order by the
    // combine; gate/up chunks write fp32 sums that a fixup kernel adds in
    // order before the SiLU product.
    const bool few_tiles = dense && per_group <= 96.0;
    P.few_tiles = few_tiles;
    P.gu = mx ? gemm_shape_mx(per_group, wide_gu)
              : few_tiles ? gemm_shape_few(T, wide_gu) : gemm_shape(per_group, wide_gu);
    P.dn = mx ? gemm_shape_mx(per_group, wide_dn)
              : few_tiles ? gemm_shape_few(T, wide_dn) : gemm_shape(per_group, wide_dn);
    P.dn_ksplit = P.gu_ksplit = 1;
    const int gu_mt = cdiv(T, P.gu.BM), gu_tiles = gu_mt * (2 * P.Fs / P.gu.BN);
    P.gu_whole = gu_tiles;
    if (few_tiles && T > 0) {
      plan_gateup_split(gu_tiles, gu_mt, P.D / 64, gemm_wgs_per_cu(P.gu), &P.gu_whole,
                        &P.gu_ksplit);
      P.dn_ksplit = ksplit_for(cdiv(T, P.dn.BM) * (P.D / P.dn.BN), P.Fs / 64,
                               gemm_wgs_per_cu(P.dn));
    }
    P.gu_shared_n = P.gu_whole + (gu_tiles - P.gu_whole) * P.gu_ksplit;
    P.gu_pc0 = (P.gu_whole / (gu_mt > 0 ? gu_mt : 1)) * (P.gu.BN / 2);
    P.gu_pw = P.gu_ksplit > 1 ? P.Fs - P.gu_pc0 : 0;
    // tile-list capacity: routed tiles plus the shared (or dense) group's (group E)
    P.gu_cap = (dense ? 0 : desc_cap(A, P.E, P.gu, 2 * P.F / P.gu.BN)) + P.gu_shared_n;
    P.dn_cap = (dense ? 0 : desc_cap(A, P.E, P.dn, P.D / P.dn.BN)) +
               cdiv(T, P.dn.BM) * (P.D / P.dn.BN) * P.dn_ksplit;
  } else {
    P.ksplit = 1; P.kchunk = P.D;
    P.gu = P.dn = GemmShape{0, 0};
    P.gu_cap = P.dn_cap = 0;
    P.few_tiles = false;
    P.dn_ksplit = P.gu_ksplit = 1;
    P.gu_whole = P.gu_shared_n = P.gu_pc0 = P.gu_pw = 0;
  }

  const size_t act = bf16 ? 2 : 4;
  const size_t hid = mx ? 1 : act;  // bytes per hidden element (E4M3 codes for MXFP8)
  size_t o = 0;
  auto take = [&](size_t bytes) { size_t at = o; o = align_up(o + bytes); return at; };
  P.xnorm = take(P.norm_weight ? (size_t)T * P.D * act : 0);
  P.partial = take(dense ? 0 : (size_t)P.ksplit * T * P.E * 4);
  P.idx = take((size_t)A * 4);
  P.w = take((size_t)A * 4);
  P.masks = take((size_t)P.ntiles * P.E * 8);
  P.tile_base = take((size_t)P.ntiles * P.E * 4);
  P.counts = take((size_t)P.E * 4);
  P.offsets = take((size_t)(P.E + 1) * 4);
  P.gu_count = take(4);
  P.dn_count = take(4);
  P.gu_desc = take((size_t)P.gu_cap * sizeof(TileDesc));
  P.dn_desc = take((size_t)P.dn_cap * sizeof(TileDesc));
  P.row_assign = take((size_t)A * 4);
  P.row_w = take((size_t)A * 4);
  P.H = take((size_t)A * P.F * hid);
  P.Hs = take((size_t)T * P.Fs * hid);
  // [T][k+ks][D]: slots k .. k+ks-1 hold the shared expert (ks K chunks)
  P.Y = take((size_t)T * (P.k + P.dn_ksplit) * P.D * 4);
  // gate and up sums of the shared group's K chunks (gate/up K split only)
  P.Pgu = take(P.gu_ksplit > 1 ? (size_t)P.gu_ksplit * T * 2 * P.gu_pw * 4 : 0);
  P.xq = take(mx ? (size_t)T * P.D : 0);        // MXFP8 input codes and scales
  P.xs = take(mx ? (size_t)T * P.D / 32 : 0);
  P.xsp = take(mx ? (size_t)A * P.D / 32 : 0);  // input scales in expert-row order
  P.Hsc = take(mx ? (size_t)A * P.F / 32 : 0);  // MXFP8 hidden-row scales
  P.Hssc = take(mx ? (size_t)T * P.Fs / 32 : 0);
  P.total = T == 0 ? 0 : o;
  return GLM_MOE_OK;
}

bool misaligned(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15) != 0; }

int check_ptr(const void* p, const char* name) {
  if (!p) return fail(GLM_MOE_EINVAL, "%s is null", name);
  if (misaligned(p)) return fail(GLM_MOE_EINVAL, "%s is not 16-byte aligned", name);
  return GLM_MOE_OK;
}

int check_ws(const Plan& P, void* ws, size_t bytes) {
  if (bytes < P.total)
    return fail(GLM_MOE_EWORKSPACE, "workspace %zu bytes < %zu needed", bytes, P.total);
  if (!ws) return fail(GLM_MOE_EINVAL, "workspace is null");
  if (reinterpret_cast<uintptr_t>(ws) % kAlign)
    return fail(GLM_MOE_EINVAL, "workspace is not %zu-byte aligned", kAlign);
  return GLM_MOE_OK;
}

template <class T>
T* at(void* ws, size_t off) { return reinterpret_cast<T*>(static_cast<char*>(ws) + off); }

}  // namespace

struct glm_moe_trace {
  int max_calls = 0;
  int calls = 0;
  std::vector<hipEvent_t> ev;  // max_calls x (GLM_MOE_NUM_STAGES + 1)
};

namespace {

struct Recorder {
  glm_moe_trace* tr;
  hipStream_t s;
  int call;
  explicit Recorder(glm_moe_trace* t, hipStream_t st) : tr(t), s(st), call(-1) {
    if (tr && tr->calls < tr->max_calls) call = tr->calls++;
  }
  hipError_t mark(int i) {
    if (call < 0) return hipSuccess;
    return hipEventRecord(tr->ev[(size_t)call * (GLM_MOE_NUM_STAGES + 1) + i], s);
  }
};

#define GLM_HIP(expr)                                                             \
  do {                                                                            \
    hipError_t e_ = (expr);                                                       \
    if (e_ != hipSuccess)                                                         \
      return fail(GLM_MOE_EHIP, "%s: %s", #expr, hipGetErrorString(e_));          \
  } while (0)

// RMSNorm of the residual stream into the workspace when requested; returns
// the input the layer runs on.
int layer_input(const Plan& P, const void* x, void* ws, hipStream_t s, const void** xin) {
  *xin = x;
  if (P.norm_weight) {
    void* xn = at<char>(ws, P.xnorm);
    GLM_HIP(launch_rmsnorm(x, P.norm_weight, xn, P.T, P.D, P.norm_eps, P.bf16, s));
    *xin = xn;
  }
  return GLM_MOE_OK;
}

int run_router(const Plan& P, const void* xin, const float* router_w, void* ws, hipStream_t s) {
  float* partial = at<float>(ws, P.partial);
  uint64_t* masks = at<uint64_t>(ws, P.masks);
  if (P.bf16)
    GLM_HIP(launch_router_logits_bf16(static_cast<const bf16_t*>(xin), router_w, partial, P.T,
                                      P.D, P.E, P.ksplit, P.kchunk, masks, s));
  else
    GLM_HIP(launch_router_logits_f32(static_cast<const float*>(xin), router_w, partial, P.T,
                                     P.D, P.E, masks, s));
  return GLM_MOE_OK;
}

int run_topk(const Plan& P, const float* corr_bias, float scale, int32_t* idx, float* w,
             void* ws, hipStream_t s) {
  GLM_HIP(launch_router_topk(at<float>(ws, P.partial), P.ksplit, corr_bias, P.T, P.E, P.k, scale,
                             P.gr, idx, w, at<uint64_t>(ws, P.masks), s));
  return GLM_MOE_OK;
}

// Expert weights of one call (the scales only for MXFP8).
struct Weights {
  const void* w1; const void* w3; const void* w2;
  const void* sw1; const void* sw3; const void* sw2;
  const uint8_t* w1s = nullptr; const uint8_t* w3s = nullptr; const uint8_t* w2s = nullptr;
  const uint8_t* sw1s = nullptr; const uint8_t* sw3s = nullptr; const uint8_t* sw2s = nullptr;
};

// Everything after the routing: permutation, grouped GEMMs, combine.
int run_experts(const Plan& P, const void* x, const void* xin, int32_t* idx, float* wts,
                const Weights& W, float* out, void* ws, hipStream_t s, Recorder& rec) {
  const void *w1 = W.w1, *w3 = W.w3, *w2 = W.w2;
  const void *shared_w1 = W.sw1, *shared_w3 = W.sw3, *shared_w2 = W.sw2;
  uint64_t* masks = at<uint64_t>(ws, P.masks);
  int32_t* tile_base = at<int32_t>(ws, P.tile_base);
  int32_t* counts = at<int32_t>(ws, P.counts);
  int32_t* offsets = at<int32_t>(ws, P.offsets);
  int32_t* gu_count = at<int32_t>(ws, P.gu_count);
  int32_t* dn_count = at<int32_t>(ws, P.dn_count);
  TileDesc* gu_desc = at<TileDesc>(ws, P.gu_desc);
  TileDesc* dn_desc = at<TileDesc>(ws, P.dn_desc);
  int32_t* row_assign = at<int32_t>(ws, P.row_assign);
  float* row_w = at<float>(ws, P.row_w);
  float* Y = at<float>(ws, P.Y);
  const void* residual = P.add_residual ? x : nullptr;

  ScanParams sp;
  sp.T = P.T; sp.E = P.E; sp.k = P.k; sp.F = P.F; sp.Fs = P.Fs; sp.D = P.D;
  // the fp32 path does not use the tile lists; give the scan a harmless shape
  sp.gu = P.bf16 ? P.gu : GemmShape{16, 128};
  sp.dn = P.bf16 ? P.dn : GemmShape{16, 128};
  sp.gu_desc_cap = P.gu_cap;
  sp.dn_desc_cap = P.dn_cap;
  sp.dn_ksplit = P.dn_ksplit;
  sp.gu_ksplit = P.gu_ksplit;
  sp.gu_whole = P.gu_whole;
  sp.gu_shared_n = P.gu_shared_n;
  // routed bf16 layers: the longest-first lists are zipped by dispatch rounds
  // (the XCD blocks below), so each XCD alternates heavy and light rounds
  const bool zip = P.bf16 && !P.mx && !P.dense;
  sp.gu_zip = zip && (GLM_ZIP & 1) ? (P.gu.BM == 256 ? kXcdBlockRoutedGu : kXcdBlock) : 0;
  sp.dn_zip = zip && (GLM_ZIP & 2) ? (P.dn.BM == 32 ? kXcdBlockDecodeDn : kXcdBlock) : 0;
  GLM_HIP(rec.mark(GLM_MOE_STAGE_SCAN));
  GLM_HIP(launch_scan(masks, sp, counts, offsets, tile_base, gu_desc, gu_count, dn_desc, dn_count, s));
  GLM_HIP(rec.mark(GLM_MOE_STAGE_SCATTER));
  if (!P.dense) GLM_HIP(launch_scatter(idx, masks, tile_base, wts, P.T, P.E, P.k, row_assign, row_w, s));

  if (P.mx) {
    uint8_t* xq = at<uint8_t>(ws, P.xq);
    uint8_t* xs = at<uint8_t>(ws, P.xs);
    GLM_HIP(rec.mark(GLM_MOE_STAGE_GATE_UP));
    uint8_t* xsp = at<uint8_t>(ws, P.xsp);
    GLM_HIP(launch_quantize_mx(static_cast<const bf16_t*>(xin), xq, xs, P.T, P.D, s));
    GLM_HIP(launch_permute_mx_scales(xs, row_assign, P.T, P.k, P.D, xsp, s));
    MxGateUpArgs ga{};
    ga.xq = xq; ga.xs = xs; ga.xsp = xsp;
    ga.row_assign = row_assign;
    ga.w1 = static_cast<const uint8_t*>(w1); ga.w1s = W.w1s;
    ga.w3 = static_cast<const uint8_t*>(w3); ga.w3s = W.w3s;
    ga.sw1 = static_cast<const uint8_t*>(shared_w1); ga.sw1s = W.sw1s;
    ga.sw3 = static_cast<const uint8_t*>(shared_w3); ga.sw3s = W.sw3s;
    ga.desc = gu_desc; ga.desc_count = gu_count;
    ga.H = at<uint8_t>(ws, P.H); ga.Hsc = at<uint8_t>(ws, P.Hsc);
    ga.Hs = at<uint8_t>(ws, P.Hs); ga.Hssc = at<uint8_t>(ws, P.Hssc);
    ga.T = P.T; ga.D = P.D; ga.E = P.E; ga.F = P.F; ga.Fs = P.Fs; ga.k = P.k;
    ga.xblk = P.gu.BM == 256 ? kXcdBlockMxGu : kXcdBlock;
    ga.grid = xcd_grid(P.gu_cap, ga.xblk);
    GLM_HIP(launch_gateup_mx(ga, P.gu, s));

    MxDownArgs da{};
    da.H = ga.H; da.Hsc = ga.Hsc; da.Hs = ga.Hs; da.Hssc = ga.Hssc;
    da.row_assign = row_assign;
    da.w2 = static_cast<const uint8_t*>(w2); da.w2s = W.w2s;
    da.sw2 = static_cast<const uint8_t*>(shared_w2); da.sw2s = W.sw2s;
    da.row_w = row_w; da.desc = dn_desc; da.desc_count = dn_count; da.Y = Y;
    da.T = P.T; da.D = P.D; da.E = P.E; da.F = P.F; da.Fs = P.Fs; da.k = P.k;
    da.xblk = P.dn.BM == 256 ? kXcdBlockMxDn : kXcdBlock;
    da.grid = xcd_grid(P.dn_cap, da.xblk);
    GLM_HIP(rec.mark(GLM_MOE_STAGE_DOWN));
    GLM_HIP(launch_down_mx(da, P.dn, s));

    GLM_HIP(rec.mark(GLM_MOE_STAGE_SHARED_COMBINE));
    GLM_HIP(launch_combine(Y, out, P.T, P.D, P.k, residual, true, s));
  } else if (P.bf16) {
    GateUpArgs ga{};
    ga.x = static_cast<const bf16_t*>(xin);
    ga.row_assign = row_assign;
    ga.w1 = static_cast<const bf16_t*>(w1); ga.w3 = static_cast<const bf16_t*>(w3);
    ga.sw1 = static_cast<const bf16_t*>(shared_w1); ga.sw3 = static_cast<const bf16_t*>(shared_w3);
    ga.desc = gu_desc; ga.desc_count = gu_count;
    ga.H = at<bf16_t>(ws, P.H); ga.Hs = at<bf16_t>(ws, P.Hs);
    ga.T = P.T; ga.D = P.D; ga.E = P.E; ga.F = P.F; ga.Fs = P.Fs; ga.k = P.k;
    // (few tiles of a dense layer: listed round-robin over the XCDs, so every
    // XCD gets the same share of whole tiles and K chunks)
    ga.xblk = P.few_tiles ? GLM_XCD_BLOCK_FEW
              : (!P.dense && P.gu.BM == 256) ? kXcdBlockRoutedGu : kXcdBlock;
    // Copy ahead of the wait on moderately filled 256-row tiles; at higher
    // average fill the second stage in flight congests the L2 miss path.
    ga.early = !P.dense && (double)P.T * P.k <= GLM_EARLY_MAX_ROWS * P.E;
    ga.ksplit = P.gu_ksplit;
    ga.P = at<float>(ws, P.Pgu);
    ga.pc0 = P.gu_pc0;
    ga.pw = P.gu_pw;
    ga.grid = xcd_grid(P.gu_cap, ga.xblk);
    GLM_HIP(rec.mark(GLM_MOE_STAGE_GATE_UP));
    GLM_HIP(launch_gateup_bf16(ga, P.gu, s));
    if (P.gu_ksplit > 1)
      GLM_HIP(launch_gateup_fixup(ga.P, ga.Hs, P.T, P.Fs, P.gu_pc0, P.gu_pw, P.gu_ksplit, s));

    DownArgs da{};
    da.H = ga.H; da.Hs = ga.Hs; da.row_assign = row_assign;
    da.w2 = static_cast<const bf16_t*>(w2); da.sw2 = static_cast<const bf16_t*>(shared_w2);
    da.row_w = row_w; da.desc = dn_desc; da.desc_count = dn_count; da.Y = Y;
    da.T = P.T; da.D = P.D; da.E = P.E; da.F = P.F; da.Fs = P.Fs; da.k = P.k;
    da.ksplit = P.dn_ksplit;
    da.xblk = P.few_tiles ? GLM_XCD_BLOCK_FEW : P.dn.BM == 32 ? kXcdBlockDecodeDn : kXcdBlock;
    da.early = ga.early;  // same two-stage ring, same fill rule
    da.grid = xcd_grid(P.dn_cap, da.xblk);
    GLM_HIP(rec.mark(GLM_MOE_STAGE_DOWN));
    GLM_HIP(launch_down_bf16(da, P.dn, s));

    GLM_HIP(rec.mark(GLM_MOE_STAGE_SHARED_COMBINE));
    // every slot of Y, in order (the shared expert's K chunks included)
    GLM_HIP(launch_combine(Y, out, P.T, P.D, P.k + P.dn_ksplit - 1, residual, true, s));
  } else {
    F32Args fa{};
    fa.x = static_cast<const float*>(xin);
    fa.row_assign = row_assign; fa.offsets = offsets;
    fa.w1 = static_cast<const float*>(w1); fa.w3 = static_cast<const float*>(w3);
    fa.w2 = static_cast<const float*>(w2);
    fa.sw1 = static_cast<const float*>(shared_w1); fa.sw3 = static_cast<const float*>(shared_w3);
    fa.sw2 = static_cast<const float*>(shared_w2);
    fa.topk_w = wts;
    fa.H = at<float>(ws, P.H); fa.Hs = at<float>(ws, P.Hs); fa.Y = Y; fa.out = out;
    fa.residual = static_cast<const float*>(residual);
    fa.T = P.T; fa.D = P.D; fa.E = P.E; fa.F = P.F; fa.Fs = P.Fs; fa.k = P.k;
    GLM_HIP(rec.mark(GLM_MOE_STAGE_GATE_UP));
    GLM_HIP(launch_gateup_f32(fa, s));
    GLM_HIP(rec.mark(GLM_MOE_STAGE_DOWN));
    GLM_HIP(launch_down_f32(fa, s));
    GLM_HIP(rec.mark(GLM_MOE_STAGE_SHARED_COMBINE));
    GLM_HIP(launch_shared_combine_f32(fa, s));
  }
  GLM_HIP(rec.mark(GLM_MOE_NUM_STAGES));
  return GLM_MOE_OK;
}

// The whole layer after argument checks: [norm ->] router -> top-k -> experts.
int run_layer(const Plan& P, const void* x, const float* router_w, const float* corr_bias,
              const Weights& W, float scale, float* out, int32_t* topk_idx_out,
              float* topk_w_out, void* workspace, hipStream_t stream, glm_moe_trace* trace) {
  int st;
  void* ws = workspace;
  hipStream_t s = stream;
  Recorder rec(trace, s);
  int32_t* idx = topk_idx_out ? topk_idx_out : at<int32_t>(ws, P.idx);
  float* wts = topk_w_out ? topk_w_out : at<float>(ws, P.w);
  GLM_HIP(rec.mark(GLM_MOE_STAGE_NORM));
  const void* xin;
  if ((st = layer_input(P, x, ws, s, &xin))) return st;
  GLM_HIP(rec.mark(GLM_MOE_STAGE_ROUTER_LOGITS));
  if ((st = run_router(P, xin, router_w, ws, s))) return st;
  GLM_HIP(rec.mark(GLM_MOE_STAGE_ROUTER_TOPK));
  if ((st = run_topk(P, corr_bias, scale, idx, wts, ws, s))) return st;
  return run_experts(P, x, xin, idx, wts, W, out, ws, s, rec);
}

int check_route_args(const void* x, const float* router_w, const float* corr_bias) {
  int st;
  if ((st = check_ptr(x, "x"))) return st;
  if ((st = check_ptr(router_w, "router_w"))) return st;
  if ((st = check_ptr(corr_bias, "corr_bias"))) return st;
  return GLM_MOE_OK;
}

}  // namespace

extern "C" {

int glm_moe_workspace_size_ex(const glm_moe_dims* d, const glm_moe_options* opts, int top_k,
                              size_t* bytes) {
  if (!bytes) return fail(GLM_MOE_EINVAL, "bytes is null");
  Plan P;
  int st = make_plan(d, top_k, opts, false, &P);
  if (st) return st;
  *bytes = P.total;
  return GLM_MOE_OK;
}

int glm_moe_workspace_size(const glm_moe_dims* d, int top_k, size_t* bytes) {
  return glm_moe_workspace_size_ex(d, nullptr, top_k, bytes);
}

int glm_moe_hidden_layout_of(const glm_moe_dims* d, const glm_moe_options* opts, int top_k,
                             glm_moe_hidden_layout* layout) {
  if (!layout) return fail(GLM_MOE_EINVAL, "layout is null");
  Plan P;
  int st = make_plan(d, top_k, opts, false, &P);
  if (st) return st;
  layout->row_assign = P.row_assign;
  layout->hidden = P.H;
  layout->hidden_scale = P.mx ? P.Hsc : 0;
  layout->shared_hidden = P.Hs;
  layout->shared_hidden_scale = P.mx ? P.Hssc : 0;
  return GLM_MOE_OK;
}

size_t glm_moe_workspace_bytes(const glm_moe_dims* d, int top_k) {
  g_err[0] = 0;
  size_t n = 0;
  if (glm_moe_workspace_size_ex(d, nullptr, top_k, &n) != GLM_MOE_OK) return 0;
  return n;
}

int glm_moe_route_ex(const glm_moe_dims* d, const glm_moe_options* opts, const void* x,
                     const float* router_w, const float* corr_bias, int top_k, float scale,
                     int32_t* topk_idx, float* topk_w, void* workspace, size_t workspace_bytes,
                     hipStream_t stream) {
  Plan P;
  int st = make_plan(d, top_k, opts, false, &P);
  if (st) return st;
  if (P.T == 0) return GLM_MOE_OK;
  if ((st = check_route_args(x, router_w, corr_bias))) return st;
  if ((st = check_ptr(topk_idx, "topk_idx"))) return st;
  if ((st = check_ptr(topk_w, "topk_w"))) return st;
  if ((st = check_ws(P, workspace, workspace_bytes))) return st;
  const void* xin;
  if ((st = layer_input(P, x, workspace, stream, &xin))) return st;
  if ((st = run_router(P, xin, router_w, workspace, stream))) return st;
  return run_topk(P, corr_bias, scale, topk_idx, topk_w, workspace, stream);
}

int glm_moe_route(const glm_moe_dims* d, const void* x, const float* router_w,
                  const float* corr_bias, int top_k, float scale, int32_t* topk_idx,
                  float* topk_w, void* workspace, size_t workspace_bytes, hipStream_t stream) {
  return glm_moe_route_ex(d, nullptr, x, router_w, corr_bias, top_k, scale, topk_idx, topk_w,
                          workspace, workspace_bytes, stream);
}

int glm_moe_forward_ex(const glm_moe_dims* d, const glm_moe_options* opts, const void* x,
                       const float* router_w, const float* corr_bias, const void* w1,
                       const void* w3, const void* w2, const void* shared_w1,
                       const void* shared_w3, const void* shared_w2, int top_k, float scale,
                       float* out, int32_t* topk_idx_out, float* topk_w_out, void* workspace,
                       size_t workspace_bytes, hipStream_t stream, glm_moe_trace* trace) {
  Plan P;
  int st = make_plan(d, top_k, opts, false, &P);
  if (st) return st;
  if (P.T == 0) return GLM_MOE_OK;
  if ((st = check_route_args(x, router_w, corr_bias))) return st;
  if ((st = check_ptr(w1, "w1")) || (st = check_ptr(w3, "w3")) || (st = check_ptr(w2, "w2")) ||
      (st = check_ptr(shared_w1, "shared_w1")) || (st = check_ptr(shared_w3, "shared_w3")) ||
      (st = check_ptr(shared_w2, "shared_w2")) || (st = check_ptr(out, "out")))
    return st;
  if (topk_idx_out && misaligned(topk_idx_out))
    return fail(GLM_MOE_EINVAL, "topk_idx_out is not 16-byte aligned");
  if (topk_w_out && misaligned(topk_w_out))
    return fail(GLM_MOE_EINVAL, "topk_w_out is not 16-byte aligned");
  if (P.mx)
    return fail(GLM_MOE_EINVAL, "MXFP8 weights take glm_moe_forward_mx (they carry scales)");
  if ((st = check_ws(P, workspace, workspace_bytes))) return st;
  Weights W{w1, w3, w2, shared_w1, shared_w3, shared_w2};
  return run_layer(P, x, router_w, corr_bias, W, scale, out, topk_idx_out, topk_w_out,
                   workspace, stream, trace);
}

int glm_moe_forward_mx(const glm_moe_dims* d, const glm_moe_options* opts, const void* x,
                       const float* router_w, const float* corr_bias, const glm_moe_mx_weights* w,
                       int top_k, float scale, float* out, int32_t* topk_idx_out,
                       float* topk_w_out, void* workspace, size_t workspace_bytes,
                       hipStream_t stream, glm_moe_trace* trace) {
  Plan P;
  int st = make_plan(d, top_k, opts, false, &P);
  if (st) return st;
  if (!P.mx)
    return fail(GLM_MOE_EINVAL, "glm_moe_forward_mx needs act_dtype BF16 and weight_dtype MXFP8");
  if (P.T == 0) return GLM_MOE_OK;
  if (!w) return fail(GLM_MOE_EINVAL, "weights is null");
  if ((st = check_route_args(x, router_w, corr_bias))) return st;
  if ((st = check_ptr(w->w1, "w1")) || (st = check_ptr(w->w1_scale, "w1_scale")) ||
      (st = check_ptr(w->w3, "w3")) || (st = check_ptr(w->w3_scale, "w3_scale")) ||
      (st = check_ptr(w->w2, "w2")) || (st = check_ptr(w->w2_scale, "w2_scale")) ||
      (st = check_ptr(w->shared_w1, "shared_w1")) ||
      (st = check_ptr(w->shared_w1_scale, "shared_w1_scale")) ||
      (st = check_ptr(w->shared_w3, "shared_w3")) ||
      (st = check_ptr(w->shared_w3_scale, "shared_w3_scale")) ||
      (st = check_ptr(w->shared_w2, "shared_w2")) ||
      (st = check_ptr(w->shared_w2_scale, "shared_w2_scale")) || (st = check_ptr(out, "out")))
    return st;
  if (topk_idx_out && misaligned(topk_idx_out))
    return fail(GLM_MOE_EINVAL, "topk_idx_out is not 16-byte aligned");
  if (topk_w_out && misaligned(topk_w_out))
    return fail(GLM_MOE_EINVAL, "topk_w_out is not 16-byte aligned");
  if ((st = check_ws(P, workspace, workspace_bytes))) return st;
  Weights W{w->w1, w->w3, w->w2, w->shared_w1, w->shared_w3, w->shared_w2,
            static_cast<const uint8_t*>(w->w1_scale), static_cast<const uint8_t*>(w->w3_scale),
            static_cast<const uint8_t*>(w->w2_scale),
            static_cast<const uint8_t*>(w->shared_w1_scale),
            static_cast<const uint8_t*>(w->shared_w3_scale),
            static_cast<const uint8_t*>(w->shared_w2_scale)};
  return run_layer(P, x, router_w, corr_bias, W, scale, out, topk_idx_out, topk_w_out,
                   workspace, stream, trace);
}

int glm_moe_mx_pack_scales(const void* src, void* dst, int64_t n_mats, int N, int K,
                           hipStream_t stream) {
  if (n_mats < 0 || N <= 0 || K <= 0 || K % 128)
    return fail(GLM_MOE_EINVAL, "bad sizes n_mats=%lld N=%d K=%d (K a multiple of 128)",
                (long long)n_mats, N, K);
  if (n_mats == 0) return GLM_MOE_OK;
  int st;
  if ((st = check_ptr(src, "src")) || (st = check_ptr(dst, "dst"))) return st;
  const size_t bytes = (size_t)n_mats * N * (K / 32);
  const uintptr_t a = reinterpret_cast<uintptr_t>(src), b = reinterpret_cast<uintptr_t>(dst);
  if (a < b + bytes && b < a + bytes) return fail(GLM_MOE_EINVAL, "src and dst overlap");
  GLM_HIP(launch_pack_mx_scales(static_cast<const uint8_t*>(src), static_cast<uint8_t*>(dst),
                                (size_t)n_mats, N, K, stream));
  return GLM_MOE_OK;
}

int glm_moe_forward_traced(const glm_moe_dims* d, const void* x, const float* router_w,
                           const float* corr_bias, const void* w1, const void* w3,
                           const void* w2, const void* shared_w1, const void* shared_w3,
                           const void* shared_w2, int top_k, float scale, float* out,
                           int32_t* topk_idx_out, float* topk_w_out, void* workspace,
                           size_t workspace_bytes, hipStream_t stream, glm_moe_trace* trace) {
  return glm_moe_forward_ex(d, nullptr, x, router_w, corr_bias, w1, w3, w2, shared_w1, shared_w3,
                            shared_w2, top_k, scale, out, topk_idx_out, topk_w_out, workspace,
                            workspace_bytes, stream, trace);
}

int glm_moe_forward(const glm_moe_dims* d, const void* x, const float* router_w,
                    const float* corr_bias, const void* w1, const void* w3, const void* w2,
                    const void* shared_w1, const void* shared_w3, const void* shared_w2,
                    int top_k, float scale, float* out, int32_t* topk_idx_out,
                    float* topk_w_out, void* workspace, size_t workspace_bytes,
                    hipStream_t stream) {
  return glm_moe_forward_ex(d, nullptr, x, router_w, corr_bias, w1, w3, w2, shared_w1, shared_w3,
                            shared_w2, top_k, scale, out, topk_idx_out, topk_w_out, workspace,
                            workspace_bytes, stream, nullptr);
}

int glm_moe_dense_workspace_size(const glm_moe_dims* d, const glm_moe_options* opts,
                                 size_t* bytes) {
  if (!bytes) return fail(GLM_MOE_EINVAL, "bytes is null");
  Plan P;
  int st = make_plan(d, 0, opts, true, &P);
  if (st) return st;
  *bytes = P.total;
  return GLM_MOE_OK;
}

int glm_moe_dense_ffn(const glm_moe_dims* d, const glm_moe_options* opts, const void* x,
                      const void* w1, const void* w3, const void* w2, float* out,
                      void* workspace, size_t workspace_bytes, hipStream_t stream,
                      glm_moe_trace* trace) {
  Plan P;
  int st = make_plan(d, 0, opts, true, &P);
  if (st) return st;
  if (P.T == 0) return GLM_MOE_OK;
  if ((st = check_ptr(x, "x")) || (st = check_ptr(w1, "w1")) || (st = check_ptr(w3, "w3")) ||
      (st = check_ptr(w2, "w2")) || (st = check_ptr(out, "out")))
    return st;
  if ((st = check_ws(P, workspace, workspace_bytes))) return st;
  Recorder rec(trace, stream);
  GLM_HIP(rec.mark(GLM_MOE_STAGE_NORM));
  const void* xin;
  if ((st = layer_input(P, x, workspace, stream, &xin))) return st;
  GLM_HIP(rec.mark(GLM_MOE_STAGE_ROUTER_LOGITS));
  GLM_HIP(rec.mark(GLM_MOE_STAGE_ROUTER_TOPK));
  Weights W{nullptr, nullptr, nullptr, w1, w3, w2};
  return run_experts(P, x, xin, nullptr, nullptr, W, out, workspace, stream, rec);
}

int glm_moe_trace_create(glm_moe_trace** trace, int max_calls) {
  if (!trace) return fail(GLM_MOE_EINVAL, "trace is null");
  if (max_calls < 1) return fail(GLM_MOE_EINVAL, "max_calls=%d < 1", max_calls);
  glm_moe_trace* t = new (std::nothrow) glm_moe_trace;
  if (!t) return fail(GLM_MOE_EINVAL, "out of host memory");
  t->max_calls = max_calls;
  t->ev.assign((size_t)max_calls * (GLM_MOE_NUM_STAGES + 1), nullptr);
  for (auto& e : t->ev) {
    hipError_t r = hipEventCreate(&e);
    if (r != hipSuccess) {
      glm_moe_trace_destroy(t);
      return fail(GLM_MOE_EHIP, "hipEventCreate: %s", hipGetErrorString(r));
    }
  }
  *trace = t;
  return GLM_MOE_OK;
}

int glm_moe_trace_destroy(glm_moe_trace* trace) {
  if (!trace) return GLM_MOE_OK;
  for (auto& e : trace->ev)
    if (e) (void)hipEventDestroy(e);
  delete trace;
  return GLM_MOE_OK;
}

int glm_moe_trace_reset(glm_moe_trace* trace) {
  if (!trace) return fail(GLM_MOE_EINVAL, "trace is null");
  trace->calls = 0;
  return GLM_MOE_OK;
}

int glm_moe_trace_read(glm_moe_trace* trace, float* stage_ms, int* calls) {
  if (!trace || !stage_ms || !calls) return fail(GLM_MOE_EINVAL, "null argument");
  for (int s = 0; s < GLM_MOE_NUM_STAGES; ++s) stage_ms[s] = 0.f;
  const int n = GLM_MOE_NUM_STAGES + 1;
  for (int c = 0; c < trace->calls; ++c) {
    hipEvent_t* ev = &trace->ev[(size_t)c * n];
    hipError_t r = hipEventSynchronize(ev[n - 1]);
    if (r != hipSuccess) return fail(GLM_MOE_EHIP, "hipEventSynchronize: %s", hipGetErrorString(r));
    for (int s = 0; s < GLM_MOE_NUM_STAGES; ++s) {
      float ms = 0.f;
      r = hipEventElapsedTime(&ms, ev[s], ev[s + 1]);
      if (r != hipSuccess) return fail(GLM_MOE_EHIP, "hipEventElapsedTime: %s", hipGetErrorString(r));
      stage_ms[s] += ms;
    }
  }
  *calls = trace->calls;
  return GLM_MOE_OK;
}

// Workspace of glm_moe_forward_noalloc: one array per GPU, resident until
// the process ends.  Host code never uses the array's name as an address:
// its device address comes from hipGetSymbolAddress, once per device.
static constexpr size_t kScratchBytes = size_t(64) << 20;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

namespace {
constexpr int kMaxDevices = 64;
std::once_flag g_scratch_once[kMaxDevices];
void* g_scratch_ptr[kMaxDevices];
hipError_t g_scratch_err[kMaxDevices];
}  // namespace

int glm_moe_forward_noalloc(const glm_moe_dims* d, const void* x, const float* router_w,
                            const float* corr_bias, const void* w1, const void* w3, const void* w2,
                            const void* shared_w1, const void* shared_w3, const void* shared_w2,
                            int top_k, float scale, float* out, int32_t* topk_idx_out,
                            float* topk_w_out, hipStream_t stream) {
  Plan P;
  int st = make_plan(d, top_k, nullptr, false, &P);
  if (st) return st;
  if (P.T == 0) return GLM_MOE_OK;
  if (P.total > kScratchBytes)
    return fail(GLM_MOE_EWORKSPACE,
                "glm_moe_forward_noalloc: these sizes need %zu bytes of workspace, above its "
                "fixed %zu-byte buffer (use glm_moe_forward with a workspace)",
                P.total, kScratchBytes);
  int dev = 0;
  GLM_HIP(hipGetDevice(&dev));
  if (dev < 0 || dev >= kMaxDevices)
    return fail(GLM_MOE_EUNSUPPORTED, "device %d beyond %d devices", dev, kMaxDevices);
  std::call_once(g_scratch_once[dev], [dev] {
    g_scratch_err[dev] = hipGetSymbolAddress(&g_scratch_ptr[dev], HIP_SYMBOL(scratch));
  });
  if (g_scratch_err[dev] != hipSuccess)
    return fail(GLM_MOE_EHIP, "hipGetSymbolAddress(scratch): %s",
                hipGetErrorString(g_scratch_err[dev]));
  return glm_moe_forward_ex(d, nullptr, x, router_w, corr_bias, w1, w3, w2, shared_w1, shared_w3,
                            shared_w2, top_k, scale, out, topk_idx_out, topk_w_out,
                            g_scratch_ptr[dev], kScratchBytes, stream, nullptr);
}

const char* glm_moe_status_string(int status) {
  switch (status) {
    case GLM_MOE_OK: return "ok";
    case GLM_MOE_EINVAL: return "invalid argument";
    case GLM_MOE_EUNSUPPORTED: return "unsupported configuration";
    case GLM_MOE_EWORKSPACE: return "workspace too small";
    case GLM_MOE_EHIP: return "HIP runtime error";
    default: return "unknown status";
  }
}

const char* glm_moe_last_error(void) { return g_err; }

int glm_moe_version(void) { return 300; }

}  // extern "C"
