// Tile list of one grouped GEMM launch: the routed experts in ascending order, each split into
// M tiles of BM rows (mt_prefix[e] is the number of M tiles before expert e) times its N tiles with the
// M index fastest, then the shared group over all T tokens.
#pragma once
#include "common.h"
#include "kernels.h"

namespace moe {

struct TileInfo {
  int group;      // 0..E-1 routed, E shared
  int n_tile;
  int row0;       // first row of the tile within the group's rows
  int nrows;      // valid rows (1..BM)
  int rowbase;    // row of the tile's first row in the group's activation/output arrays
};

template <int BM>
__device__ __forceinline__ TileInfo decode_tile(int id, const GemmArgs& a, int nt_r, int mt_routed) {
  TileInfo ti;
  const int32_t* __restrict__ mt_prefix = a.mt_prefix;
  const int routed_tiles = mt_routed * nt_r;
  if (id < routed_tiles) {
    int lo = 0, hi = a.E;
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (mt_prefix[mid] * nt_r <= id) lo = mid;
      else hi = mid - 1;
    }
    const int e = lo;
    const int p0 = mt_prefix[e];
    const int mt = mt_prefix[e + 1] - p0;
    const int local = id - p0 * nt_r;
    ti.group = e;
    ti.n_tile = local / mt;
    const int m_tile = local - ti.n_tile * mt;
    const int o0 = a.offsets[e], n_e = a.offsets[e + 1] - o0;
    ti.row0 = m_tile * BM;
    ti.nrows = min(BM, n_e - ti.row0);
    ti.rowbase = o0 + ti.row0;
  } else {
    const int mt = cdiv(a.T, BM);
    const int local = id - routed_tiles;
    ti.group = a.E;
    ti.n_tile = local / mt;
    const int m_tile = local - ti.n_tile * mt;
    ti.row0 = m_tile * BM;
    ti.nrows = min(BM, a.T - ti.row0);
    ti.rowbase = ti.row0;
  }
  return ti;
}

// Tile id -> (group, N tile, rows), from LDS copies of mt_prefix and offsets: routed experts ascending,
// M index fastest within an expert (the M tiles of one N tile share its weight rows: blocks that take
// them together start on the same weight stream, so later ones often find it in the XCD's L2), then the
// shared group in the same order.
template <int BM>
__device__ __forceinline__ TileInfo decode_tile_lds(int id, const int32_t* mtp, const int32_t* off, int E, int T,
                                                    int nt_r, int nt_s) {
  TileInfo ti;
  const int routed_tiles = mtp[E] * nt_r;
  if (id < routed_tiles) {
    int lo = 0, hi = E;
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (mtp[mid] * nt_r <= id) lo = mid;
      else hi = mid - 1;
    }
    const int e = __builtin_amdgcn_readfirstlane(lo);
    const int local = id - mtp[e] * nt_r;
    ti.group = e;
    const int mt_e = mtp[e + 1] - mtp[e];
    ti.n_tile = local / mt_e;
    const int m_tile = local - ti.n_tile * mt_e;
    const int o0 = off[e], n_e = off[e + 1] - o0;
    ti.row0 = m_tile * BM;
    ti.nrows = min(BM, n_e - ti.row0);
    ti.rowbase = o0 + ti.row0;
  } else {
    const int local = id - routed_tiles;
    ti.group = E;
    const int mt_s = (T + BM - 1) / BM;
    ti.n_tile = local / mt_s;
    const int m_tile = local - ti.n_tile * mt_s;
    ti.row0 = m_tile * BM;
    ti.nrows = min(BM, T - ti.row0);
    ti.rowbase = ti.row0;
  }
  ti.group = __builtin_amdgcn_readfirstlane(ti.group);
  ti.n_tile = __builtin_amdgcn_readfirstlane(ti.n_tile);
  ti.row0 = __builtin_amdgcn_readfirstlane(ti.row0);
  ti.nrows = __builtin_amdgcn_readfirstlane(ti.nrows);
  ti.rowbase = __builtin_amdgcn_readfirstlane(ti.rowbase);
  return ti;
}

// Schedule of the matrix-core grouped GEMMs. The tile list (routed experts ascending, M index fastest
// within an N tile, then the shared group) is cut into eight contiguous ranges of equal estimated
// cost, one per XCD, over the first 7/8 of the total; the rest is a pool for any XCD whose range is
// done. A tile's cost follows its measured duration by valid rows (below): 100 when more
// than half of its bm rows are valid (both token halves of the block multiply), 69 or 62 otherwise (one
// half multiplies; streaming its weights still takes most of the time). Within a range the blocks of
// that XCD take tiles in order from a counter, then from the pool's.
// Exclusive prefix sum over the 512 threads of a block (buf: 512 entries of LDS, reusable on return):
// a shuffle scan within each wave, then the totals of the waves before.
__device__ __forceinline__ long long block_exclusive_scan(long long v, long long* buf) {
  const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
  long long x = v;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const long long y = __shfl_up(x, o, 64);
    if (lane >= o) x += y;
  }
  if (lane == 63) buf[wave] = x;
  __syncthreads();
  long long before = 0;
  for (int w = 0; w < wave; ++w) before += buf[w];
  __syncthreads();
  return before + x - v;
}

// One block of 512 threads, one thread per group (routed experts 0..E-1, the shared group E): its M tiles and the cost of one row
// of N tiles, then block-wide scans give every group its first tile and the cost before it, and the
// group holding a boundary's cost finds the boundary tile within itself.
__device__ __forceinline__ void schedule_mfma_block(const int32_t* __restrict__ offsets, int E, int T, int bm,
                                                         int ntr0, int nts0, int ntr1, int nts1,
                                                         int32_t* __restrict__ mt_prefix, int32_t* __restrict__ xrange,
                                                         int32_t* __restrict__ xcount) {
  __shared__ long long buf[512];
  __shared__ long long s_tot[2];
  const int g = threadIdx.x;
  const bool grp = g <= E;
  // relative duration of a tile by its valid rows (measured on the V3 layer, both projections: a tile
  // whose second half of tokens is empty skips half the MFMAs, and one of at most bm/4 rows also most
  // of the token copies; the shared group's full tiles run a little longer than routed ones)
  auto tile_cost = [&](int n, int m) {
    const int r = min(bm, n - m * bm);
    return r > bm / 2 ? (g == E ? 103 : 100) : (r > bm / 4 ? 69 : 62);
  };
  int n = 0, mt = 0, S = 0;
  if (grp) {
    n = g < E ? offsets[g + 1] - offsets[g] : T;
    mt = cdiv(n, bm);
    for (int m = 0; m < mt; ++m) S += tile_cost(n, m);
  }
  if (g < 2 * kSchedCount) xcount[g] = 0;
  // M tiles before each routed group; for g = E this is their total
  const long long mpre = block_exclusive_scan(g < E ? mt : 0, buf);
  if (grp) mt_prefix[g] = (int)mpre;
  for (int l = 0; l < 2; ++l) {
    const int nt = g < E ? (l ? ntr1 : ntr0) : (l ? nts1 : nts0);
    const long long C = grp ? (long long)nt * S : 0;       // cost of the group's tiles
    const long long ntl = grp ? (long long)nt * mt : 0;    // and their number
    const long long before = block_exclusive_scan(C, buf);
    const long long id0 = block_exclusive_scan(ntl, buf);
    if (g == E) {
      s_tot[0] = before + C;
      s_tot[1] = id0 + ntl;
    }
    __syncthreads();
    const long long total = s_tot[0];
    const long long ranged = total - total / kSchedPoolDiv;   // cost of the XCD ranges; the rest is the pool
    int32_t* r = xrange + kSchedRange * l;
    if (g == 0) {
      r[0] = 0;
      r[9] = (int)s_tot[1];
      if (ranged <= 0) r[8] = 0;
    }
    // boundary x: the first tile whose preceding cost reaches x * ranged / 8 (x = 8: the pool's start).
    // The groups with tiles split (0, total] into the intervals (before, before + C]; the owner's tiles are
    // nt equal columns of cost S (M fastest within an N column): it skips whole columns, then scans the M
    // tiles of the next one.
    for (int x = 1; x <= 8; ++x) {
      const long long tgt = ranged * x / 8;
      if (tgt <= 0) {
        if (g == 0) r[x] = 0;
        continue;
      }
      if (C > 0 && before < tgt && tgt <= before + C) {
        const long long off = tgt - before;
        const long long nf = off / S;        // whole N columns (each S) before the boundary
        long long cum = nf * S;
        int mi = 0;
        while (cum < off) cum += tile_cost(n, mi++);
        r[x] = (int)(id0 + nf * mt + mi);
      }
    }
    __syncthreads();   // s_tot is written again by the next launch's totals
  }
}

}  // namespace moe
