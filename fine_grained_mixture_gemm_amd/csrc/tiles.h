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

}  // namespace moe
