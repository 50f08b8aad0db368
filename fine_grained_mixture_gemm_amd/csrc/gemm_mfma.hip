// Grouped expert GEMMs on the gfx950 matrix cores, bf16 and E4M3.
//
// Each routed expert e owns rows offsets[e]..offsets[e+1]-1 of the dispatched order; the shared
// experts form one more group over all T tokens. One launch covers every group:
//   gate/up:  [g | v] = X W13^T, a = SiLU(g) * v        (X gathered from u through perm_src)
//   down:     y = a W2^T
// (DeepSeek Technical Report: MoE Architecture, 1.1 and 5.3 [1]; SwiGLU per the DeepSeek-V3
// walkthrough, "invariant core"). The E4M3 variant follows 3.6 of the same report: 1x128 activation
// scales, 128x128 weight scales, and every 128-element partial product multiplied by its two scales
// and added into an fp32 accumulator (promotion interval 128); the gate/up epilogue quantizes a
// again per row per 128 columns.
//
// Tile: 256 weight rows x 128 tokens, K staged 128 bytes at a time (128 E4M3 or 64 bf16 elements).
// The product is formed transposed (weights as the MFMA A operand, tokens as B) so that each lane's
// accumulators belong to one token: the token's scale is one value per lane and the 1x128 requant
// reduces over channels held by the same lane. Eight waves: each owns 64 weight rows (for gate/up:
// 32 gate channels and the same 32 up channels) against one half (64) of the tokens; weights stream
// from HBM straight into registers, tokens go through a double-buffered, XOR-swizzled LDS tile.
// The grid is persistent: blocks are split by XCD (block id mod 8) and each XCD walks one
// contiguous range of the tile list, in which neighbouring tiles share an expert's weight tile.
#include "common.h"
#include "kernels.h"
#include "tiles.h"

namespace moe {

constexpr int kBM = 128;       // tokens per tile
constexpr int kBW = 256;       // weight rows per tile
constexpr int kStageB = 128;   // K bytes per stage
#ifndef MOE_GEMM_WM
#define MOE_GEMM_WM 2
#endif
constexpr int kWM = MOE_GEMM_WM;          // token groups (waves along M)
constexpr int kThreads = 256 * kWM;       // 4 weight-row groups x kWM token groups of waves
constexpr int kTJ = 8 / kWM;              // 16-token MFMA tiles per wave
constexpr int kBQ = kBM * 8 / kThreads;   // 16-byte B chunks each thread stages per K step

template <bool FP8>
__device__ __forceinline__ void mma_stage(f32x4 (&acc)[4][kTJ], const i32x4 (&A)[4][2], const uint8_t* __restrict__ lds_b,
                                          const float* __restrict__ lds_sx, const float (&sw)[4], int lane, int tok0) {
  const int tr = lane & 15, g = lane >> 4;
#pragma unroll
  for (int j = 0; j < kTJ; ++j) {
    const int row = tok0 + 16 * j + tr;
    const int sw0 = ((g) ^ (row & 7)) * 16, sw1 = ((4 + g) ^ (row & 7)) * 16;
    const i32x4 b0 = *reinterpret_cast<const i32x4*>(lds_b + row * kStageB + sw0);
    const i32x4 b1 = *reinterpret_cast<const i32x4*>(lds_b + row * kStageB + sw1);
    if constexpr (FP8) {
      const float sx = lds_sx[row];
      const i32x8 bb = {b0[0], b0[1], b0[2], b0[3], b1[0], b1[1], b1[2], b1[3]};
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const i32x8 aa = {A[i][0][0], A[i][0][1], A[i][0][2], A[i][0][3], A[i][1][0], A[i][1][1], A[i][1][2], A[i][1][3]};
        const f32x4 zero = {0.f, 0.f, 0.f, 0.f};
        const f32x4 p = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(aa, bb, zero, 0, 0, 0, 127, 0, 127);
        const float sc = sx * sw[i];
#pragma unroll
        for (int r = 0; r < 4; ++r) acc[i][j][r] = fmaf(sc, p[r], acc[i][j][r]);
      }
    } else {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, A[i][0]),
                                                            __builtin_bit_cast(bf16x8, b0), acc[i][j], 0, 0, 0);
        acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, A[i][1]),
                                                            __builtin_bit_cast(bf16x8, b1), acc[i][j], 0, 0, 0);
      }
    }
  }
}

// LDS: two B stages (+ token scales) during the K loop; reused for the epilogue tile afterwards.
constexpr int kLdsStage = kBM * kStageB + kBM * 4;
constexpr int kLdsBytes = kBM * 512 + 4 * kBM * 4;   // >= 2 * kLdsStage; largest epilogue + amax table

template <bool FP8, bool GATEUP>
__global__ __launch_bounds__(kThreads, 1) void grouped_gemm_mfma(GemmArgs a) {
  static_assert(kLdsBytes >= 2 * kLdsStage, "lds");
  __shared__ __attribute__((aligned(16))) uint8_t lds[kLdsBytes];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wn = wave & 3, wm = wave >> 2;   // weight-row group, token half (wave-uniform)
  const int tok0 = 16 * kTJ * wm;
  const int esz = FP8 ? 1 : 2;
  const int32_t* __restrict__ mt_prefix = a.mt_prefix;
  const int mt_routed = mt_prefix[a.E];
  const int fr = a.f, fs = a.fs;
  const int nt_r = GATEUP ? fr / 128 : a.d / kBW;
  const int nt_s = GATEUP ? fs / 128 : a.d / kBW;
  const int total = mt_routed * nt_r + (fs > 0 ? cdiv(a.T, kBM) * nt_s : 0);

  const int xcd = blockIdx.x & 7, slot = blockIdx.x >> 3, per = gridDim.x >> 3;
  const int chunk = cdiv(total, 8);
  const int t_begin = xcd * chunk, t_end = min(total, t_begin + chunk);

  for (int id = t_begin + slot; id < t_end; id += per) {
    const TileInfo ti = decode_tile<kBM>(id, a, nt_r, mt_routed);
    const bool shared = ti.group == a.E;
    const int fg = shared ? fs : fr;                       // inner dim of this group
    const int kelems = GATEUP ? a.d : fg;                  // reduction length
    const int kbytes = kelems * esz;
    const int nst = kbytes / kStageB;
    const int kblk = kelems / 128;                         // 128-element scale blocks along K
    // ---- operand bases (uniform) and per-lane 32-bit offsets
    const uint8_t* __restrict__ W;
    const float* __restrict__ WS = nullptr;
    if (GATEUP) {
      W = shared ? a.w_shared : a.w_routed + (size_t)ti.group * (2 * (size_t)fr) * a.d * esz;
      if (FP8) WS = shared ? a.ws_shared : a.ws_routed + (size_t)ti.group * (2 * fr / 128) * (a.d / 128);
    } else {
      W = shared ? a.w_shared : a.w_routed + (size_t)ti.group * (size_t)a.d * fr * esz;
      if (FP8) WS = shared ? a.ws_shared : a.ws_routed + (size_t)ti.group * (a.d / 128) * (fr / 128);
    }
    const uint8_t* __restrict__ X = shared ? a.x_shared : a.x_routed;
    const float* __restrict__ XS = FP8 ? (shared ? a.xs_shared : a.xs_routed) : nullptr;
    const int c0 = ti.n_tile * (GATEUP ? 128 : kBW);
    // first weight row of each of this wave's four 16-row tiles (uniform)
    int wrow0[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      if (GATEUP) wrow0[i] = (i < 2 ? c0 : fg + c0) + 32 * wn + 16 * (i & 1);
      else wrow0[i] = c0 + 64 * wn + 16 * i;
    }
    uint32_t aoff[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) aoff[i] = (uint32_t)(wrow0[i] + (lane & 15)) * kbytes + 16 * (lane >> 4);
    // weight block-scale rows: gate/up tiles 0,1 share one 128-row block and 2,3 another; the down
    // tiles all lie in one block
    const float* __restrict__ wsA = FP8 ? WS + (size_t)(wrow0[0] / 128) * kblk : nullptr;
    const float* __restrict__ wsB = FP8 ? WS + (size_t)(wrow0[2] / 128) * kblk : nullptr;
    // ---- token rows this thread stages (2 x 16-byte chunks per stage) and its scale row
    auto src_row = [&](int r) -> int {
      const int rr = min(r, ti.nrows - 1);
      if (GATEUP) return shared ? ti.rowbase + rr : a.perm_src[ti.rowbase + rr];
      return ti.rowbase + rr;
    };
    uint32_t boff[kBQ];
#pragma unroll
    for (int q = 0; q < kBQ; ++q) {
      const int id16 = q * kThreads + tid;
      boff[q] = (uint32_t)src_row(id16 >> 3) * kbytes + (id16 & 7) * 16;
    }
    const uint32_t sxoff = (FP8 && tid < kBM) ? (uint32_t)src_row(tid) * kblk : 0u;

    f32x4 acc[4][kTJ];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < kTJ; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

    i32x4 Acur[4][2], Anxt[4][2];
    i32x4 Bst[kBQ];
    float sxst = 0.f;
    float swA_nxt = 1.f, swB_nxt = 1.f;
    auto load_a = [&](i32x4 (&A)[4][2], int kb) {
      const uint8_t* Wk = W + kb * kStageB;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        A[i][0] = *reinterpret_cast<const i32x4*>(Wk + aoff[i]);
        A[i][1] = *reinterpret_cast<const i32x4*>(Wk + aoff[i] + 64);
      }
    };
    auto load_b = [&](int kb) {
      const uint8_t* Xk = X + kb * kStageB;
#pragma unroll
      for (int q = 0; q < kBQ; ++q) Bst[q] = *reinterpret_cast<const i32x4*>(Xk + boff[q]);
      if (FP8 && tid < kBM) sxst = XS[sxoff + kb];
    };
    auto store_b = [&](int buf) {
      uint8_t* base = lds + buf * kLdsStage;
#pragma unroll
      for (int q = 0; q < kBQ; ++q) {
        const int id16 = q * kThreads + tid;
        const int row = id16 >> 3, c = id16 & 7;
        *reinterpret_cast<i32x4*>(base + row * kStageB + ((c ^ (row & 7)) * 16)) = Bst[q];
      }
      if (FP8 && tid < kBM) reinterpret_cast<float*>(base + kBM * kStageB)[tid] = sxst;
    };
    auto load_scales = [&](int kb) {
      if constexpr (FP8) {
        swA_nxt = wsA[kb];
        swB_nxt = GATEUP ? wsB[kb] : swA_nxt;
      }
    };

    load_b(0);
    load_a(Acur, 0);
    load_scales(0);
    for (int kb = 0; kb < nst; ++kb) {
      uint8_t* buf = lds + (kb & 1) * kLdsStage;
      store_b(kb & 1);
      const float sw[4] = {swA_nxt, swA_nxt, swB_nxt, swB_nxt};
      __syncthreads();
      if (kb + 1 < nst) {
        load_scales(kb + 1);
        load_b(kb + 1);
        load_a(Anxt, kb + 1);
      }
      mma_stage<FP8>(acc, Acur, buf, reinterpret_cast<const float*>(buf + kBM * kStageB), sw, lane, tok0);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        Acur[i][0] = Anxt[i][0];
        Acur[i][1] = Anxt[i][1];
      }
    }
    __syncthreads();   // LDS is reused by the epilogue

    // ---- epilogue. Lane holds, for token tok0 + 16j + (lane & 15), weight-row channels 4 (lane >> 4) + r
    // of each 16-row tile i.
    const int tr = lane & 15, g4 = 4 * (lane >> 4);
    if constexpr (GATEUP) {
      float av[2][kTJ][4];
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < kTJ; ++j)
#pragma unroll
          for (int r = 0; r < 4; ++r) av[i][j][r] = silu(acc[i][j][r]) * acc[i + 2][j][r];
      const size_t out_stride = (size_t)fg * esz;           // bytes per output row
      uint8_t* OUT = (shared ? a.out_shared : a.out_routed) + (size_t)ti.rowbase * out_stride + (size_t)c0 * esz;
      if constexpr (FP8) {
        float* red = reinterpret_cast<float*>(lds + kBM * 128);   // [4 weight-row groups][128 tokens]
        float inv[kTJ];
#pragma unroll
        for (int j = 0; j < kTJ; ++j) {
          float m = 0.f;
#pragma unroll
          for (int i = 0; i < 2; ++i)
#pragma unroll
            for (int r = 0; r < 4; ++r) m = fmaxf(m, fabsf(av[i][j][r]));
          m = fmaxf(m, __shfl_xor(m, 16, 64));
          m = fmaxf(m, __shfl_xor(m, 32, 64));
          if (lane < 16) red[wn * kBM + tok0 + 16 * j + tr] = m;
        }
        __syncthreads();
        float* OS = (shared ? a.out_scale_shared : a.out_scale_routed);
#pragma unroll
        for (int j = 0; j < kTJ; ++j) {
          const int tok = tok0 + 16 * j + tr;
          const float m = fmaxf(fmaxf(red[tok], red[kBM + tok]), fmaxf(red[2 * kBM + tok], red[3 * kBM + tok]));
          float s;
          e4m3_scales(m, s, inv[j]);
          if (wn == 0 && lane < 16 && tok < ti.nrows) OS[(size_t)(ti.rowbase + tok) * (fg / 128) + ti.n_tile] = s;
        }
#pragma unroll
        for (int j = 0; j < kTJ; ++j)
#pragma unroll
          for (int i = 0; i < 2; ++i) {
            const int tok = tok0 + 16 * j + tr, ch = 32 * wn + 16 * i + g4;
            const uint32_t qv = f32x4_to_e4m3x4(av[i][j][0] * inv[j], av[i][j][1] * inv[j], av[i][j][2] * inv[j],
                                                av[i][j][3] * inv[j]);
            *reinterpret_cast<uint32_t*>(lds + tok * 128 + ch) = qv;
          }
        __syncthreads();
#pragma unroll
        for (int q = 0; q < kBM * 8 / kThreads; ++q) {
          const int id16 = q * kThreads + tid, row = id16 >> 3, c = id16 & 7;
          if (row < ti.nrows)
            *reinterpret_cast<uint4*>(OUT + (size_t)row * out_stride + c * 16) =
                *reinterpret_cast<const uint4*>(lds + row * 128 + c * 16);
        }
      } else {
#pragma unroll
        for (int j = 0; j < kTJ; ++j)
#pragma unroll
          for (int i = 0; i < 2; ++i) {
            const int tok = tok0 + 16 * j + tr, ch = 32 * wn + 16 * i + g4;
            uint2 v;
            v.x = uint32_t(f32_to_bf16(av[i][j][0])) | (uint32_t(f32_to_bf16(av[i][j][1])) << 16);
            v.y = uint32_t(f32_to_bf16(av[i][j][2])) | (uint32_t(f32_to_bf16(av[i][j][3])) << 16);
            *reinterpret_cast<uint2*>(lds + tok * 256 + ch * 2) = v;
          }
        __syncthreads();
#pragma unroll
        for (int q = 0; q < kBM * 16 / kThreads; ++q) {
          const int id16 = q * kThreads + tid, row = id16 >> 4, c = id16 & 15;
          if (row < ti.nrows)
            *reinterpret_cast<uint4*>(OUT + (size_t)row * out_stride + c * 16) =
                *reinterpret_cast<const uint4*>(lds + row * 256 + c * 16);
        }
      }
    } else if constexpr (!FP8) {
      // y in fp32: each lane stores its 4 consecutive channels of one token (16 bytes)
      const size_t out_stride = (size_t)a.d * 4;
      uint8_t* OUT = (shared ? a.out_shared : a.out_routed) + (size_t)ti.rowbase * out_stride + (size_t)c0 * 4;
#pragma unroll
      for (int j = 0; j < kTJ; ++j) {
        const int tok = tok0 + 16 * j + tr;
        if (tok < ti.nrows) {
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int ch = 64 * wn + 16 * i + g4;
            *reinterpret_cast<f32x4*>(OUT + (size_t)tok * out_stride + ch * 4) = acc[i][j];
          }
        }
      }
    } else {
      // y tile in bf16 (the combine payload of the E4M3 path): 128 tokens x 256 channels through LDS
      const size_t out_stride = (size_t)a.d * 2;
      uint8_t* OUT = (shared ? a.out_shared : a.out_routed) + (size_t)ti.rowbase * out_stride + (size_t)c0 * 2;
#pragma unroll
      for (int j = 0; j < kTJ; ++j)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int tok = tok0 + 16 * j + tr, ch = 64 * wn + 16 * i + g4;
          uint2 v;
          v.x = uint32_t(f32_to_bf16(acc[i][j][0])) | (uint32_t(f32_to_bf16(acc[i][j][1])) << 16);
          v.y = uint32_t(f32_to_bf16(acc[i][j][2])) | (uint32_t(f32_to_bf16(acc[i][j][3])) << 16);
          *reinterpret_cast<uint2*>(lds + tok * 512 + ch * 2) = v;
        }
      __syncthreads();
#pragma unroll
      for (int q = 0; q < kBM * 32 / kThreads; ++q) {
        const int id16 = q * kThreads + tid, row = id16 >> 5, c = id16 & 31;
        if (row < ti.nrows)
          *reinterpret_cast<uint4*>(OUT + (size_t)row * out_stride + c * 16) =
              *reinterpret_cast<const uint4*>(lds + row * 512 + c * 16);
      }
    }
    __syncthreads();   // epilogue LDS reads finish before the next tile's stage 0 store
  }
}

int gemm_mfma_bm() { return kBM; }

hipError_t launch_gemm_mfma(const GemmArgs& a, bool fp8, bool gateup, int grid, hipStream_t s) {
  if (fp8) {
    if (gateup) grouped_gemm_mfma<true, true><<<grid, kThreads, 0, s>>>(a);
    else grouped_gemm_mfma<true, false><<<grid, kThreads, 0, s>>>(a);
  } else {
    if (gateup) grouped_gemm_mfma<false, true><<<grid, kThreads, 0, s>>>(a);
    else grouped_gemm_mfma<false, false><<<grid, kThreads, 0, s>>>(a);
  }
  return hipGetLastError();
}

}  // namespace moe
