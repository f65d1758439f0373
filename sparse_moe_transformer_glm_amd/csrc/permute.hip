// Token permutation of the GLM-5.2 MoE layer: group the (token, slot)
// assignments by expert so each expert's tokens form contiguous rows.  Rows of
// one expert are in ascending token order (a stable counting sort), which makes
// the whole layer deterministic.
#include "common.h"

namespace glm {
namespace {

constexpr int kScanThreads = 1024;
constexpr int kParts = kScanThreads / kMaxExperts;  // token-tile ranges scanned in parallel

#ifndef GLM_BLK_M
#define GLM_BLK_M 8
#endif
#ifndef GLM_BLK_N
#define GLM_BLK_N 4
#endif
// Position `local` of a group's tile list -> (row tile m, column tile nt).
// Routed groups (shared == false) hold few row tiles: column-tile major, row
// tiles inner.  The shared (or dense) group's tiles all cost the same, so the
// workgroups running together stay in step; they are listed in blocks of
// GLM_BLK_M row tiles x GLM_BLK_N column tiles, so that the tiles running
// together on one XCD read few distinct operand panels through its L2.
__device__ inline void tile_order(int local, int mt, int nt_all, bool shared, int* m, int* nt) {
  if (!shared) {
    *nt = local / mt;
    *m = local % mt;
    return;
  }
  const int bm = min(GLM_BLK_M, mt), bn = GLM_BLK_N;
  const int band = local / (bm * nt_all);          // band of bm row tiles
  const int hb = min(bm, mt - band * bm);          // rows in this band
  const int rem = local - band * bm * nt_all;
  const int cb = rem / (hb * bn);                  // column block within the band
  const int wb = min(bn, nt_all - cb * bn);        // columns in this block
  const int r2 = rem - cb * hb * bn;
  *m = band * bm + r2 % hb;
  *nt = cb * bn + r2 / hb;
}

// First row of row tile m of a group of `rows` rows cut into mt tiles of at
// most BM rows.  The rows are dealt out evenly in units of `gran` rows (the
// MFMA row blocks of both wave rows): the tiles sharing a weight slice do
// nearly the same work and stay in step, and no tile computes more MFMA row
// blocks than the group needs.
__device__ inline int tile_row0(int m, int mt, int rows, int gran) {
  const int units = cdiv(rows, gran);
  return min(rows, (int)(((long long)m * units) / mt) * gran);
}

// Tile descriptors of one GEMM, positions [0, total).  Listing position lo
// (0..E) holds group og[lo], whose tiles start at position pos[lo]; pos is
// non-decreasing and groups without tiles repeat the next group's position.
// Wave w writes a contiguous chunk of positions, 64 consecutive ones per round
// (coalesced 16-byte stores).  One binary search finds the group of the chunk's
// first position; after that each lane steps forward from the group of the
// previous round's last position, a few LDS reads per round.
__device__ inline void write_descs(const int* pos, const int* og, int total, const int* cnt,
                                   const int* off, int T, int E, int BM, int shared_nt,
                                   int col_w, int ksplit, int whole, int zip_xb,
                                   TileDesc* __restrict__ out) {
  constexpr int kWaves = kScanThreads / kWave;
  const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x / kWave;
  const int unit = xcd_round(zip_xb > 0 ? total : 0, zip_xb);  // tiles per zipped unit
  const int chunk = cdiv(cdiv(total, kWaves), kWave) * kWave;
  const int b0 = wave * chunk, b1 = min(total, b0 + chunk);
  if (b0 >= b1) return;
  int lo = 0, hi = E;  // largest position with pos <= b0
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (pos[mid] <= b0) lo = mid; else hi = mid - 1;
  }
  for (int base = b0; base < b1; base += kWave) {
    const int i = base + lane;
    int l = lo;
    while (l < E && pos[l + 1] <= i) ++l;
    lo = __shfl(l, kWave - 1, kWave);
    if (i >= b1) continue;
    const int g = og[l];
    const int rows = g < E ? cnt[g] : T;
    const int mt = cdiv(rows, BM);
    int nt, m, r0, rt, kc = 0, chunk = 0;
    if (mt == 1 && g < E) {  // one row tile (the common case): no divisions
      m = 0;
      nt = i - pos[l];
      r0 = 0;
      rt = rows;
    } else {
      if (g == E && whole >= 0) {
        // gate/up of the shared group: `whole` tiles, then the others in
        // `ksplit` K chunks (chunk innermost), tiles column-tile major
        const int li = i - pos[l];
        int t = li;
        if (li >= whole) {
          t = whole + (li - whole) / ksplit;
          kc = (li - whole) % ksplit;
          chunk = kChunkTile;
        }
        nt = t / mt;
        m = t % mt;
      } else {
        // the shared group's K chunks count as extra column tiles (chunk innermost)
        const int ks = g == E ? ksplit : 1;
        tile_order(i - pos[l], mt, shared_nt * ks, g == E, &m, &nt);
        kc = nt % ks;
        nt /= ks;
      }
      const int gran = min(64, BM);
      r0 = tile_row0(m, mt, rows, gran);
      rt = tile_row0(m + 1, mt, rows, gran) - r0;
    }
    TileDesc d;
    d.group = g | (mt == 1 ? kSoleRowTile : 0) | chunk | (kc << kKChunkShift);
    d.row0 = (g < E ? off[g] : 0) + r0;
    d.rows = rt;
    d.col0 = nt * col_w;
    out[zip_position(i, total, unit)] = d;
  }
}

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

  // Per expert: count, then exclusive prefix sums of the counts and of the
  // tile counts of both GEMMs over the 256 expert slots (a wave scan per 64
  // experts, then the wave totals).
  __shared__ int s_wsum[kMaxExperts / kWave][3];
  int c = 0, v_gu = 0, v_dn = 0;
  if (tid < kMaxExperts) {
#pragma unroll
    for (int i = 0; i < kParts; ++i) c += part[i][tid];
    s_cnt[tid] = c;
    if (tid < E) {
      v_gu = cdiv(c, p.gu.BM) * (2 * p.F / p.gu.BN);
      v_dn = cdiv(c, p.dn.BM) * (p.D / p.dn.BN);
    } else {
      c = 0;
    }
    const int lane = tid & (kWave - 1);
    int i0 = c, i1 = v_gu, i2 = v_dn;  // inclusive sums within the wave
#pragma unroll
    for (int d = 1; d < kWave; d <<= 1) {
      const int a0 = __shfl_up(i0, d, kWave), a1 = __shfl_up(i1, d, kWave),
                a2 = __shfl_up(i2, d, kWave);
      if (lane >= d) { i0 += a0; i1 += a1; i2 += a2; }
    }
    if (lane == kWave - 1) {
      s_wsum[tid / kWave][0] = i0;
      s_wsum[tid / kWave][1] = i1;
      s_wsum[tid / kWave][2] = i2;
    }
    // keep the exclusive values until the wave totals are known
    c = i0 - c;
    v_gu = i1 - v_gu;
    v_dn = i2 - v_dn;
  }
  __syncthreads();
  if (tid < kMaxExperts) {
    for (int w = 0; w < tid / kWave; ++w) {
      c += s_wsum[w][0];
      v_gu += s_wsum[w][1];
      v_dn += s_wsum[w][2];
    }
    if (tid <= E) {  // slot E holds the totals over the routed experts
      s_off[tid] = c;
      s_gu[tid] = v_gu;
      s_dn[tid] = v_dn;
    }
  }
  __syncthreads();
  if (tid == 0) {
    if (E == kMaxExperts) {  // no slot E above: totals from the wave sums
      int o = 0, gsum = 0, dsum = 0;
      for (int w = 0; w < kMaxExperts / kWave; ++w) {
        o += s_wsum[w][0];
        gsum += s_wsum[w][1];
        dsum += s_wsum[w][2];
      }
      s_off[E] = o;
      s_gu[E] = gsum;
      s_dn[E] = dsum;
    }
    // the shared expert is group E of both GEMMs, over every token
    s_gu[E + 1] = min(s_gu[E] + p.gu_shared_n, p.gu_desc_cap);
    s_dn[E + 1] = min(s_dn[E] + cdiv(p.T, p.dn.BM) * (p.D / p.dn.BN) * p.dn_ksplit,
                      p.dn_desc_cap);
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

  // Listing order of the groups.  With row tiles of more than 32 rows: the
  // shared expert first, then the routed experts by rows per row tile, most
  // first (ties: lower index), so the longest tiles start first and the
  // shortest end the launch, which keeps the CUs' last tiles short.  Decode
  // tiles (32 rows) all cost about one weight slice, so there the routed
  // experts keep index order and the shared expert comes last.  s_pg / s_pd:
  // first tile of the group listed at position p; s_og / s_od: that group.
  __shared__ int s_pg[kMaxExperts + 1], s_og[kMaxExperts + 1];
  __shared__ int s_pd[kMaxExperts + 1], s_od[kMaxExperts + 1];
  // sort keys (rows per row tile, then the index, packed into one int so all
  // keys differ) and tile counts of every routed group
  __shared__ int s_kg[kMaxExperts], s_kd[kMaxExperts], s_tg[kMaxExperts], s_td[kMaxExperts];
  // per group: rank and first tile in each list, summed over kParts slices
  __shared__ int s_rank[4][kMaxExperts];
  const bool lpt_g = p.gu.BM > 32, lpt_d = p.dn.BM > 32;
  if (tid < kMaxExperts) {
    const int c = tid < E ? s_cnt[tid] : 0;
    const int mg = cdiv(c, p.gu.BM), md = cdiv(c, p.dn.BM);
    s_kg[tid] = ((c == 0 ? 0 : c / mg) << 16) | (0xFFFF - tid);
    s_kd[tid] = ((c == 0 ? 0 : c / md) << 16) | (0xFFFF - tid);
    s_tg[tid] = mg * (2 * p.F / p.gu.BN);
    s_td[tid] = md * (p.D / p.dn.BN);
    s_rank[0][tid] = 0; s_rank[1][tid] = 0; s_rank[2][tid] = 0; s_rank[3][tid] = 0;
  }
  __syncthreads();
  {
    // thread (e, q) compares group e with the groups of slice q
    const int per_q = cdiv(E, kParts), f0 = q * per_q, f1 = min(E, f0 + per_q);
    if ((lpt_g || lpt_d) && e < E && f0 < f1) {
      const int kg = s_kg[e], kd = s_kd[e];
      int rg = 0, rd = 0, bg = 0, bd = 0;
#pragma unroll 8
      for (int f = f0; f < f1; ++f) {
        if (s_kg[f] > kg) { ++rg; bg += s_tg[f]; }
        if (s_kd[f] > kd) { ++rd; bd += s_td[f]; }
      }
      atomicAdd(&s_rank[0][e], rg);
      atomicAdd(&s_rank[1][e], bg);
      atomicAdd(&s_rank[2][e], rd);
      atomicAdd(&s_rank[3][e], bd);
    }
  }
  __syncthreads();
  if (tid < E) {
    if (lpt_g) {
      const int rg = s_rank[0][tid];
      s_og[1 + rg] = tid;  // after the shared group's tiles:
      s_pg[1 + rg] = p.gu_shared_n + s_rank[1][tid];
    } else {
      s_og[tid] = tid;
      s_pg[tid] = s_gu[tid];
    }
    if (lpt_d) {
      const int rd = s_rank[2][tid];
      s_od[1 + rd] = tid;
      s_pd[1 + rd] = cdiv(p.T, p.dn.BM) * (p.D / p.dn.BN) * p.dn_ksplit + s_rank[3][tid];
    } else {
      s_od[tid] = tid;
      s_pd[tid] = s_dn[tid];
    }
  }
  if (tid == 0) {
    s_og[lpt_g ? 0 : E] = E;
    s_pg[lpt_g ? 0 : E] = lpt_g ? 0 : s_gu[E];
    s_od[lpt_d ? 0 : E] = E;
    s_pd[lpt_d ? 0 : E] = lpt_d ? 0 : s_dn[E];
  }
  __syncthreads();

  // tile descriptors: groups in listing order, then output-column tile, then row tile
  write_descs(s_pg, s_og, s_gu[E + 1], s_cnt, s_off, p.T, E, p.gu.BM, 2 * p.Fs / p.gu.BN,
              p.gu.BN / 2, p.gu_ksplit, p.gu_ksplit > 1 ? p.gu_whole : -1,
              lpt_g ? p.gu_zip : 0, gu_desc);
  write_descs(s_pd, s_od, s_dn[E + 1], s_cnt, s_off, p.T, E, p.dn.BM, p.D / p.dn.BN, p.dn.BN,
              p.dn_ksplit, -1, lpt_d ? p.dn_zip : 0, dn_desc);
}

// One wave per 64-token tile.  A token's rank among the tile's tokens of
// expert e is the number of lower lanes whose mask bit is set.
__global__ __launch_bounds__(64) void scatter_kernel(
    const int32_t* __restrict__ topk_idx, const uint64_t* __restrict__ masks,
    const int32_t* __restrict__ tile_base, const float* __restrict__ topk_w, int T, int E,
    int k, int32_t* __restrict__ row_assign, float* __restrict__ row_w) {
  const int tile = blockIdx.x, lane = threadIdx.x;
  const int t = tile * kTokTile + lane;
  if (t >= T) return;
  const uint64_t below = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  for (int j = 0; j < k; ++j) {
    const int e = topk_idx[(size_t)t * k + j];
    const uint64_t m = masks[(size_t)tile * E + e];
    const int row = tile_base[(size_t)tile * E + e] + __popcll(m & below);
    row_assign[row] = t * k + j;
    row_w[row] = topk_w[(size_t)t * k + j];
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
                          const int32_t* tile_base, const float* topk_w, int T, int E, int k,
                          int32_t* row_assign, float* row_w, hipStream_t s) {
  scatter_kernel<<<cdiv(T, kTokTile), 64, 0, s>>>(topk_idx, masks, tile_base, topk_w, T, E, k,
                                                   row_assign, row_w);
  return hipGetLastError();
}

}  // namespace glm
