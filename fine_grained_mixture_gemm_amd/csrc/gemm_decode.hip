// Grouped E4M3 expert GEMMs for a decode-sized batch (at most 128 tokens, so every group holds at most
// 128 rows): the same products as gemm_mfma.hip (gate/up + SwiGLU + 1x128 requant, and down), shaped for
// streaming the touched experts' weights once at HBM rate.
//
// DeepSeek Technical Report: MoE Architecture, 1.1 (shared + routed experts), 3.6 (E4M3 with 1x128
// activation and 128x128 weight scales, every 128-element partial product scaled and added into fp32);
// SwiGLU per the DeepSeek-V3 walkthrough, "invariant core".
//
// With a handful of rows per expert there is no weight reuse to exploit: the work is a weight stream.
// One block per (group, 128-channel tile): gate/up covers gate channels c0..c0+127 and the same up
// channels (256 weight rows), down covers output rows c0..c0+127. Each of the 8 waves owns 16 of those
// channels (gate/up: its 16 gate rows and the matching 16 up rows) for the group's rows, taken in passes
// of kDecJ 16-token MFMA tiles (only tiles that hold rows are loaded and multiplied). Weights and
// tokens go straight from global memory into registers in the MFMA operand layout (lane: row lane % 16,
// 16-byte chunks g and 4 + g of the 128-byte K block, g = lane / 16), with kDecP K blocks in flight per
// wave; all loads are plain vector loads, so the compiler's wait counts stay exact. The token rows are
// the same for the 8 waves of a block and come from the vector L1 after the first wave. Weights in the
// tiled layout (pack_weights in gemm_mfma.hip) are read as 1 KB contiguous per load instruction.
#include "common.h"
#include "kernels.h"

#include <utility>

namespace moe {

constexpr int kDecWaves = 8;
constexpr int kDecThreads = 64 * kDecWaves;
// 16-token tiles per pass over the weights (a group with more rows takes several passes) and K blocks in
// flight per wave. One tile and two blocks measured best for both projections at the V3 decode shape
// (the 64-row shared group then takes four passes, which is why it starts first).
constexpr int kDecJG = 1, kDecPG = 2, kDecJD = 1, kDecPD = 2;

template <bool GATEUP, int J>
struct DecStage {
  static constexpr int NA = GATEUP ? 2 : 1;
  i32x8 a[NA];         // weight rows: gate, up (gate/up) or the down rows
  i32x8 b[J];          // token rows of the live 16-token tiles
  float sx[J];         // their E4M3 scales
  float ws[NA];        // weight block scales
};

__device__ __forceinline__ i32x8 load_k_block(const uint8_t* row_k, int g) {
  const i32x4 lo = *reinterpret_cast<const i32x4*>(row_k + 16 * g);
  const i32x4 hi = *reinterpret_cast<const i32x4*>(row_k + 64 + 16 * g);
  return i32x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
}

template <bool GATEUP, int kDecJ, int kDecP, bool PACKED>
__global__ __launch_bounds__(kDecThreads) void grouped_gemm_decode(GemmArgs a) {
  using Stage = DecStage<GATEUP, kDecJ>;
  constexpr int NA = Stage::NA;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int tr = lane & 15, g = lane >> 4;
  const int E = a.E;

  // ---- block -> (group, 128-channel tile). The shared group comes first: it has the most rows (all T
  // tokens), so its blocks take several passes and should not be the last ones to start.
  const int nt_r = GATEUP ? a.f / 128 : a.d / 128;
  const int nt_s = a.fs > 0 ? (GATEUP ? a.fs / 128 : a.d / 128) : 0;
  const int id = (int)blockIdx.x - nt_s;
  const int group = id < 0 ? E : id / nt_r;
  const int nt = id < 0 ? id + nt_s : id - group * nt_r;
  const bool shared = group == E;
  const int row0 = shared ? 0 : a.offsets[group];
  const int n = shared ? a.T : a.offsets[group + 1] - row0;
  if (n <= 0) return;
  const int fg = shared ? a.fs : a.f;              // inner dim of the group
  const int K = GATEUP ? a.d : fg;                 // reduction length (E4M3 bytes)
  const int nkb = K / 128;
  const int c0 = nt * 128;

  // ---- weights: rows of this wave, as byte offsets from the group's weight block
  const uint8_t* W;
  const float* WS;
  if (GATEUP) {
    W = shared ? a.w_shared : a.w_routed + (size_t)group * (2 * (size_t)a.f) * a.d;
    WS = shared ? a.ws_shared : a.ws_routed + (size_t)group * (2 * a.f / 128) * (a.d / 128);
  } else {
    W = shared ? a.w_shared : a.w_routed + (size_t)group * (size_t)a.d * a.f;
    WS = shared ? a.ws_shared : a.ws_routed + (size_t)group * (a.d / 128) * (a.f / 128);
  }
  uint32_t woff[NA];
  int wbrow[NA];                                   // weight block row of each operand
  if constexpr (PACKED) {
    // tiled layout: the 16-row block of this wave in stage 0 of its 256-row tile (gate/up: tile nt, gate
    // block wave, up block 8 + wave; down: tile nt / 2, block 8 (nt % 2) + wave), lane-contiguous
    const int tile = GATEUP ? nt : nt >> 1;
    const int blk = GATEUP ? wave : 8 * (nt & 1) + wave;
    woff[0] = ((uint32_t)tile * nkb << 15) + blk * 2048 + lane * 16;
    if constexpr (GATEUP) woff[1] = woff[0] + 8 * 2048;
  } else {
    woff[0] = (uint32_t)(c0 + 16 * wave + tr) * K;
    if constexpr (GATEUP) woff[1] = (uint32_t)(fg + c0 + 16 * wave + tr) * K;
  }
  wbrow[0] = nt;
  if constexpr (GATEUP) wbrow[1] = fg / 128 + nt;

  const uint8_t* X = shared ? a.x_shared : a.x_routed;
  const float* XS = shared ? a.xs_shared : a.xs_routed;
  for (int rp = 0; rp < n; rp += 16 * kDecJ) {
  // ---- tokens of this pass: row of each 16-token tile for this lane (rows past n repeat the last row)
  const int J = min(kDecJ, (n - rp + 15) >> 4);
  uint32_t xrow[kDecJ];
#pragma unroll
  for (int j = 0; j < kDecJ; ++j) {
    const int r = min(rp + 16 * j + tr, n - 1);
    xrow[j] = GATEUP ? (shared ? r : a.perm_src[row0 + r]) : (shared ? r : row0 + r);
  }

  Stage st[kDecP];
  auto load = [&](Stage& s, int kb) {
#pragma unroll
    for (int t = 0; t < NA; ++t) {
      if constexpr (PACKED) {
        const uint8_t* p = W + woff[t] + ((size_t)kb << 15);
        const i32x4 lo = *reinterpret_cast<const i32x4*>(p);
        const i32x4 hi = *reinterpret_cast<const i32x4*>(p + 1024);
        s.a[t] = i32x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
      } else {
        s.a[t] = load_k_block(W + woff[t] + (size_t)kb * 128, g);
      }
      s.ws[t] = WS[(size_t)wbrow[t] * nkb + kb];
    }
#pragma unroll
    for (int j = 0; j < kDecJ; ++j) {
      if (j < J) {
        s.b[j] = load_k_block(X + (size_t)xrow[j] * K + (size_t)kb * 128, g);
        s.sx[j] = XS[(size_t)xrow[j] * nkb + kb];
      }
    }
  };

  f32x4 acc[NA][kDecJ];
#pragma unroll
  for (int t = 0; t < NA; ++t)
#pragma unroll
    for (int j = 0; j < kDecJ; ++j) acc[t][j] = f32x4{0.f, 0.f, 0.f, 0.f};
  const f32x4 zero = {0.f, 0.f, 0.f, 0.f};
  auto compute = [&](const Stage& s) {
#pragma unroll
    for (int j = 0; j < kDecJ; ++j) {
      if (j < J) {
#pragma unroll
        for (int t = 0; t < NA; ++t) {
          const f32x4 p = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(s.a[t], s.b[j], zero, 0, 0, 0, 127, 0, 127);
          acc[t][j] += (s.sx[j] * s.ws[t]) * p;
        }
      }
    }
  };

#pragma unroll
  for (int p = 0; p < kDecP; ++p)
    if (p < nkb) load(st[p], p);
  for (int k0 = 0; k0 < nkb; k0 += kDecP) {
#pragma unroll
    for (int p = 0; p < kDecP; ++p) {
      const int kb = k0 + p;
      if (kb < nkb) {
        compute(st[p]);
        if (kb + kDecP < nkb) load(st[p], kb + kDecP);
      }
    }
  }

  // ---- epilogue. Lane holds, for row rp + 16 j + tr of the group, channels 4 g + r of the wave's 16.
  if constexpr (GATEUP) {
    __shared__ float red[kDecWaves][16 * kDecJ];
    float av[kDecJ][4];
#pragma unroll
    for (int j = 0; j < kDecJ; ++j) {
      float m = 0.f;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        av[j][r] = silu(acc[0][j][r]) * acc[1][j][r];
        m = fmaxf(m, fabsf(av[j][r]));
      }
      m = fmaxf(m, __shfl_xor(m, 16, 64));
      m = fmaxf(m, __shfl_xor(m, 32, 64));
      if (lane < 16) red[wave][16 * j + tr] = m;
    }
    __syncthreads();
    uint8_t* OUT = shared ? a.out_shared : a.out_routed;
    float* OS = shared ? a.out_scale_shared : a.out_scale_routed;
    const int orow0 = shared ? 0 : row0;
#pragma unroll
    for (int j = 0; j < kDecJ; ++j) {
      const int r = rp + 16 * j + tr;
      if (j < J && r < n) {
        float m = red[0][16 * j + tr];
#pragma unroll
        for (int w = 1; w < kDecWaves; ++w) m = fmaxf(m, red[w][16 * j + tr]);
        float s, inv;
        e4m3_scales(m, s, inv);
        const size_t orow = (size_t)(orow0 + r);
        if (wave == 0 && g == 0) OS[orow * (fg / 128) + nt] = s;
        *reinterpret_cast<uint32_t*>(OUT + orow * fg + c0 + 16 * wave + 4 * g) =
            f32x4_to_e4m3x4(av[j][0] * inv, av[j][1] * inv, av[j][2] * inv, av[j][3] * inv);
      }
    }
    __syncthreads();   // `red` is written again by the next pass
  } else {
    uint8_t* OUT = shared ? a.out_shared : a.out_routed;
    const int orow0 = shared ? 0 : row0;
#pragma unroll
    for (int j = 0; j < kDecJ; ++j) {
      const int r = rp + 16 * j + tr;
      if (j < J && r < n) {
        uint2 v;
        v.x = uint32_t(f32_to_bf16(acc[0][j][0])) | (uint32_t(f32_to_bf16(acc[0][j][1])) << 16);
        v.y = uint32_t(f32_to_bf16(acc[0][j][2])) | (uint32_t(f32_to_bf16(acc[0][j][3])) << 16);
        *reinterpret_cast<uint2*>(OUT + ((size_t)(orow0 + r) * a.d + c0 + 16 * wave + 4 * g) * 2) = v;
      }
    }
  }
  }
}

// Up to 128 tokens the weight stream of this kernel beats the tiled kernel (V3 layer: 96 tokens 1.59 vs
// 1.83 ms per step, 128 tokens 1.79 vs 1.91); at 192 it is slower (2.25 vs 2.07): groups of more than 16
// rows stream their weights once per 16-token pass.
int gemm_decode_max_tokens() { return 128; }

hipError_t launch_gemm_decode(const GemmArgs& a, bool gateup, hipStream_t s) {
  const int nt_r = gateup ? a.f / 128 : a.d / 128;
  const int nt_s = a.fs > 0 ? (gateup ? a.fs / 128 : a.d / 128) : 0;
  const int blocks = a.E * nt_r + nt_s;
  if (blocks == 0) return hipSuccess;
  if (a.packed) {
    if (gateup) grouped_gemm_decode<true, kDecJG, kDecPG, true><<<blocks, kDecThreads, 0, s>>>(a);
    else grouped_gemm_decode<false, kDecJD, kDecPD, true><<<blocks, kDecThreads, 0, s>>>(a);
  } else {
    if (gateup) grouped_gemm_decode<true, kDecJG, kDecPG, false><<<blocks, kDecThreads, 0, s>>>(a);
    else grouped_gemm_decode<false, kDecJD, kDecPD, false><<<blocks, kDecThreads, 0, s>>>(a);
  }
  return hipGetLastError();
}

}  // namespace moe
