// Token permutation of the GLM-5.2 MoE layer: group the (token, slot)
// assignments by expert so each expert's tokens form contiguous rows.  Rows of
// one expert are in ascending token order (a stable counting sort), which makes
// the whole layer deterministic.
#include "common.h"

namespace glm {
namespace {

constexpr int kScanThreads = 1024;
constexpr int kParts = kScanThreads / kMaxExperts;  // token-tile ranges scanned in parallel

// Single workgroup.  masks[tile][e] has bit i set when token tile*64+i chose e.
__global__ __launch_bounds__(kScanThreads) void scan_kernel(
    const uint64_t* __restrict__ masks, ScanParams p, int32_t* __restrict__ counts,
    int32_t* __restrict__ offsets, int32_t* __restrict__ tile_base,
    TileDesc* __restrict__ gu_desc, int32_t* __restrict__ gu_count,
    TileDesc* __restrict__ dn_desc, int32_t* __restrict__ dn_count) {
  __shared__ int part[kParts][kMaxExperts];
  __shared__ int s_cnt[kMaxExperts + 1];
  __shared__ int s_off[kMaxExperts + 1];
  __shared__ int s_gu[kMaxExperts + 2];
  __shared__ int s_dn[kMaxExperts + 2];

  const int tid = threadIdx.x;
  const int e = tid % kMaxExperts, q = tid / kMaxExperts;
  const int E = p.E;
  const int NT = cdiv(p.T, kTokTile);
  const int per = cdiv(NT, kParts);
  const int tb = min(NT, q * per), te = min(NT, tb + per);

  int sum = 0;
  if (e < E) {
#pragma unroll 8
    for (int t = tb; t < te; ++t) sum += __popcll(masks[(size_t)t * E + e]);
  }
  part[q][e] = sum;
  __syncthreads();
  if (tid < kMaxExperts) {
    int c = 0;
#pragma unroll
    for (int i = 0; i < kParts; ++i) c += part[i][tid];
    s_cnt[tid] = c;
  }
  __syncthreads();

  if (tid == 0) {
    // expert offsets and the tile counts of each group of the two GEMMs
    const int gu_nt = 2 * p.F / p.gu.BN, gu_nts = 2 * p.Fs / p.gu.BN;
    const int dn_nt = p.D / p.dn.BN;
    int off = 0, gu = 0, dn = 0;
    for (int g = 0; g < E; ++g) {
      const int c = s_cnt[g];
      s_off[g] = off;
      s_gu[g] = gu;
      s_dn[g] = dn;
      off += c;
      gu += cdiv(c, p.gu.BM) * gu_nt;
      dn += cdiv(c, p.dn.BM) * dn_nt;
    }
    s_off[E] = off;
    // the shared expert is group E of both GEMMs, over every token
    s_gu[E] = gu;
    gu += cdiv(p.T, p.gu.BM) * gu_nts;
    s_gu[E + 1] = min(gu, p.gu_desc_cap);
    s_dn[E] = dn;
    dn += cdiv(p.T, p.dn.BM) * dn_nt;
    s_dn[E + 1] = min(dn, p.dn_desc_cap);
  }
  __syncthreads();

  if (tid < E) counts[tid] = s_cnt[tid];
  if (tid <= E) offsets[tid] = s_off[tid];
  if (tid == 0) {
    *gu_count = s_gu[E + 1];
    *dn_count = s_dn[E + 1];
  }

  // row base of every (token tile, expert)
  if (e < E) {
    int base = s_off[e];
    for (int i = 0; i < q; ++i) base += part[i][e];
    for (int t = tb; t < te; ++t) {
      tile_base[(size_t)t * E + e] = base;
      base += __popcll(masks[(size_t)t * E + e]);
    }
  }

  // tile descriptors: group-major, then output-column tile, then row tile
  const int gu_total = s_gu[E + 1];
  for (int i = tid; i < gu_total; i += kScanThreads) {
    int lo = 0, hi = E;  // largest g with s_gu[g] <= i
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (s_gu[mid] <= i) lo = mid; else hi = mid - 1;
    }
    const int g = lo;
    const int rows = g < E ? s_cnt[g] : p.T;
    const int mt = cdiv(rows, p.gu.BM);
    const int local = i - s_gu[g];
    const int nt = local / mt, m = local % mt;
    TileDesc d;
    d.group = g;
    d.row0 = m * p.gu.BM;
    d.rows = min(p.gu.BM, rows - d.row0);
    d.col0 = nt * (p.gu.BN / 2);
    gu_desc[i] = d;
  }
  const int dn_total = s_dn[E + 1];
  for (int i = tid; i < dn_total; i += kScanThreads) {
    int lo = 0, hi = E;
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (s_dn[mid] <= i) lo = mid; else hi = mid - 1;
    }
    const int g = lo;
    const int grows = g < E ? s_cnt[g] : p.T;
    const int mt = cdiv(grows, p.dn.BM);
    const int local = i - s_dn[g];
    const int nt = local / mt, m = local % mt;
    TileDesc d;
    d.group = g;
    d.row0 = m * p.dn.BM;
    d.rows = min(p.dn.BM, grows - d.row0);
    d.col0 = nt * p.dn.BN;
    dn_desc[i] = d;
  }
}

// One wave per 64-token tile.  A token's rank among the tile's tokens of
// expert e is the number of lower lanes whose mask bit is set.
__global__ __launch_bounds__(64) void scatter_kernel(
    const int32_t* __restrict__ topk_idx, const uint64_t* __restrict__ masks,
    const int32_t* __restrict__ tile_base, int T, int E, int k,
    int32_t* __restrict__ row_assign) {
  const int tile = blockIdx.x, lane = threadIdx.x;
  const int t = tile * kTokTile + lane;
  if (t >= T) return;
  const uint64_t below = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  for (int j = 0; j < k; ++j) {
    const int e = topk_idx[(size_t)t * k + j];
    const uint64_t m = masks[(size_t)tile * E + e];
    const int row = tile_base[(size_t)tile * E + e] + __popcll(m & below);
    row_assign[row] = t * k + j;
  }
}

}  // namespace

hipError_t launch_scan(const uint64_t* masks, const ScanParams& p, int32_t* counts,
                       int32_t* offsets, int32_t* tile_base, TileDesc* gu_desc,
                       int32_t* gu_count, TileDesc* dn_desc, int32_t* dn_count,
                       hipStream_t s) {
  scan_kernel<<<1, kScanThreads, 0, s>>>(masks, p, counts, offsets, tile_base, gu_desc, gu_count,
                                         dn_desc, dn_count);
  return hipGetLastError();
}

hipError_t launch_scatter(const int32_t* topk_idx, const uint64_t* masks,
                          const int32_t* tile_base, int T, int E, int k, int32_t* row_assign,
                          hipStream_t s) {
  scatter_kernel<<<cdiv(T, kTokTile), 64, 0, s>>>(topk_idx, masks, tile_base, T, E, k,
                                                   row_assign);
  return hipGetLastError();
}

}  // namespace glm
