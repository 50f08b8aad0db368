// Grouped expert GEMMs in fp32 on the vector ALUs (fp32 weights), and the M-tile schedule that every
// grouped GEMM launch reads.
//   gate/up: a = SiLU(X W1^T) * (X W3^T)     down: y = a W2^T
// (DeepSeek Technical Report: MoE Architecture, 1.1; SwiGLU per the DeepSeek-V3 walkthrough, "invariant
// core"). Tiles of 64 rows x 32 channels (gate/up, both halves) or 64 x 64 (down), 16 K per step.
#include "common.h"
#include "kernels.h"
#include "tiles.h"

namespace moe {

// mt_prefix[e] = sum over e' < e of ceil(count_e' / bm), count_e = offsets[e+1] - offsets[e].
__global__ __launch_bounds__(256) void ffn_schedule(const int32_t* __restrict__ offsets, int E, int bm,
                                                    int32_t* __restrict__ mt_prefix) {
  __shared__ int32_t s_mt[256];
  const int e = threadIdx.x;
  s_mt[e] = e < E ? cdiv(offsets[e + 1] - offsets[e], bm) : 0;
  __syncthreads();
  if (e == 0) {
    int m = 0;
    for (int i = 0; i < E; ++i) {
      mt_prefix[i] = m;
      m += s_mt[i];
    }
    mt_prefix[E] = m;
  }
}

hipError_t launch_schedule(const int32_t* offsets, int E, int bm, int32_t* mt_prefix, hipStream_t s) {
  ffn_schedule<<<1, 256, 0, s>>>(offsets, E, bm, mt_prefix);
  return hipGetLastError();
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

// One thread per group (routed experts 0..E-1, the shared group E): its M tiles and the cost of one row
// of N tiles, then block-wide scans give every group its first tile and the cost before it, and the
// group holding a boundary's cost finds the boundary tile within itself.
__global__ __launch_bounds__(512) void ffn_schedule_mfma(const int32_t* __restrict__ offsets, int E, int T, int bm,
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

hipError_t launch_schedule_mfma(const int32_t* offsets, int E, int T, int bm, const int (&nt_r)[2], const int (&nt_s)[2],
                                int32_t* mt_prefix, int32_t* xrange, int32_t* xcount, hipStream_t s) {
  ffn_schedule_mfma<<<1, 512, 0, s>>>(offsets, E, T, bm, nt_r[0], nt_s[0], nt_r[1], nt_s[1], mt_prefix, xrange, xcount);
  return hipGetLastError();
}

constexpr int kSBM = 64, kSBK = 16;

template <bool GATEUP>
__global__ __launch_bounds__(256) void grouped_gemm_simt(GemmArgs a) {
  constexpr int BN = GATEUP ? 32 : 64;       // output channels per tile
  constexpr int WR = GATEUP ? 2 * BN : BN;   // weight rows per tile
  __shared__ float Xs[kSBK][kSBM + 1];
  __shared__ float Ws[kSBK][WR + 1];
  const int mt_routed = a.mt_prefix[a.E];
  const int nt_r = GATEUP ? cdiv(a.f, BN) : cdiv(a.d, BN);
  const int nt_s = GATEUP ? cdiv(a.fs, BN) : cdiv(a.d, BN);
  const int total = mt_routed * nt_r + (a.fs > 0 ? cdiv(a.T, kSBM) * nt_s : 0);
  const int id = blockIdx.x;
  if (id >= total) return;
  const TileInfo ti = decode_tile<kSBM>(id, a, nt_r, mt_routed);
  const bool shared = ti.group == a.E;
  const int fg = shared ? a.fs : a.f;
  const int K = GATEUP ? a.d : fg;
  const float* W = reinterpret_cast<const float*>(shared ? a.w_shared : a.w_routed);
  if (!shared) W += GATEUP ? (size_t)ti.group * 2 * a.f * a.d : (size_t)ti.group * a.d * a.f;
  const float* X = reinterpret_cast<const float*>(shared ? a.x_shared : a.x_routed);
  const int c0 = ti.n_tile * BN;
  const int nout = GATEUP ? fg : a.d;
  const int tid = threadIdx.x, ty = tid >> 4, tx = tid & 15;

  int xrow[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int r = min((q * 256 + tid) / kSBK, ti.nrows - 1);
    xrow[q] = (GATEUP && !shared) ? a.perm_src[ti.rowbase + r] : ti.rowbase + r;
  }
  float acc[4][4] = {};   // gate/up: [row][0..1 gate, 2..3 up]; down: [row][4 channels]
  for (int k0 = 0; k0 < K; k0 += kSBK) {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int e = q * 256 + tid, r = e / kSBK, k = e % kSBK;
      Xs[k][r] = (k0 + k < K) ? X[(size_t)xrow[q] * K + k0 + k] : 0.f;
    }
    for (int e = tid; e < WR * kSBK; e += 256) {
      const int r = e / kSBK, k = e % kSBK;
      int wr;
      bool ok;
      if (GATEUP) {
        const int ch = c0 + (r % BN);
        ok = ch < fg;
        wr = (r < BN ? 0 : fg) + ch;
      } else {
        wr = c0 + r;
        ok = wr < a.d;
      }
      Ws[k][r] = (ok && k0 + k < K) ? W[(size_t)wr * K + k0 + k] : 0.f;
    }
    __syncthreads();
#pragma unroll
    for (int k = 0; k < kSBK; ++k) {
      float x[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) x[i] = Xs[k][ty * 4 + i];
      if (GATEUP) {
        const float g0 = Ws[k][2 * tx], g1 = Ws[k][2 * tx + 1], u0 = Ws[k][BN + 2 * tx], u1 = Ws[k][BN + 2 * tx + 1];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          acc[i][0] = fmaf(x[i], g0, acc[i][0]);
          acc[i][1] = fmaf(x[i], g1, acc[i][1]);
          acc[i][2] = fmaf(x[i], u0, acc[i][2]);
          acc[i][3] = fmaf(x[i], u1, acc[i][3]);
        }
      } else {
        float w[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) w[j] = Ws[k][tx * 4 + j];
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
          for (int j = 0; j < 4; ++j) acc[i][j] = fmaf(x[i], w[j], acc[i][j]);
      }
    }
    __syncthreads();
  }
  float* OUT = reinterpret_cast<float*>(shared ? a.out_shared : a.out_routed);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int r = ty * 4 + i;
    if (r >= ti.nrows) continue;
    float* orow = OUT + (size_t)(ti.rowbase + r) * nout;
    if (GATEUP) {
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const int ch = c0 + 2 * tx + j;
        if (ch < fg) orow[ch] = silu(acc[i][j]) * acc[i][2 + j];
      }
    } else {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int ch = c0 + tx * 4 + j;
        if (ch < a.d) orow[ch] = acc[i][j];
      }
    }
  }
}

int gemm_simt_bm() { return kSBM; }

hipError_t launch_gemm_simt(const GemmArgs& a, bool gateup, int max_tiles, hipStream_t s) {
  if (max_tiles <= 0) return hipSuccess;
  if (gateup) grouped_gemm_simt<true><<<max_tiles, 256, 0, s>>>(a);
  else grouped_gemm_simt<false><<<max_tiles, 256, 0, s>>>(a);
  return hipGetLastError();
}

}  // namespace moe
