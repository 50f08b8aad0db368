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

__global__ __launch_bounds__(512) void ffn_schedule_mfma(const int32_t* __restrict__ offsets, int E, int T, int bm,
                                                         int ntr0, int nts0, int ntr1, int nts1,
                                                         int32_t* __restrict__ mt_prefix, int32_t* __restrict__ xrange,
                                                         int32_t* __restrict__ xcount) {
  schedule_mfma_block(offsets, E, T, bm, ntr0, nts0, ntr1, nts1, mt_prefix, xrange, xcount);
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
