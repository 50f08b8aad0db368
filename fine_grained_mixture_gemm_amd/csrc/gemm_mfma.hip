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
// reduces over channels held by the same lane. Four waves (one per SIMD) each own 64 weight rows (for
// gate/up: 32 gate channels and the same 32 up channels) against all 128 tokens.
// Operands move global -> LDS by the LDS-DMA loads (no registers), into a ring of three stages: two
// stages are in flight while the third is multiplied, which covers the HBM latency of the weight
// stream. LDS rows are XOR-swizzled in 16-byte chunks (chunk c of row r sits at c ^ (r & 7)), so the
// MFMA operand reads are free of bank conflicts.
// The grid is persistent: blocks are split by XCD (block id mod 8) and each XCD walks one contiguous
// range of the tile list, in which neighbouring tiles share an expert's weight tile in that XCD's L2.
#include "common.h"
#include "kernels.h"
#include "tiles.h"

namespace moe {

constexpr int kBM = 128;        // tokens per tile
constexpr int kBW = 256;        // weight rows per tile
constexpr int kStageB = 128;    // K bytes per stage
#ifndef MOE_GEMM_WM
#define MOE_GEMM_WM 2
#endif
constexpr int kWM = MOE_GEMM_WM;          // waves along the tokens (each takes 128 / kWM tokens)
constexpr int kThreads = 256 * kWM;       // 4 weight-row groups x kWM token groups
constexpr int kTJ = 8 / kWM;              // 16-token MFMA tiles per wave
constexpr int kG = kThreads / 8;          // LDS rows covered by one pass of the loader
constexpr int kStages = 3;      // LDS ring depth
constexpr int kAChunks = kBW * 8 / kThreads;   // 16-byte A chunks each thread moves per stage (8)
constexpr int kBChunks = kBM * 8 / kThreads;   // 16-byte B chunks each thread moves per stage (4)
constexpr int kSlotA = kBW * kStageB;          // 32 KB
constexpr int kSlotB = kBM * kStageB;          // 16 KB
constexpr int kSlotS = kSlotA + kSlotB;          // token scales [128] then the two weight scales
constexpr int kSlot = kSlotS + kBM * 4 + 16;
constexpr int kLdsBytes = kStages * kSlot;
static_assert(kLdsBytes >= kBM * 512 + 4 * kBM * 4, "the epilogue reuses the ring");

typedef __attribute__((address_space(3))) void* lds_ptr_t;

// Global -> LDS copy of 16 (or 4) bytes per lane; the wave writes 64 consecutive pieces at `lds_base`.
__device__ __forceinline__ void dma16(const void* src, uint8_t* lds_base) {
  __builtin_amdgcn_global_load_lds(src, (lds_ptr_t)lds_base, 16, 0, 0);
}
__device__ __forceinline__ void dma4(const void* src, uint8_t* lds_base) {
  __builtin_amdgcn_global_load_lds(src, (lds_ptr_t)lds_base, 4, 0, 0);
}

// Wait until at most N vector-memory operations of this wave are outstanding (gfx9 s_waitcnt fields:
// vmcnt[3:0] | expcnt[6:4] | lgkmcnt[11:8] | vmcnt_hi[15:14]; expcnt and lgkmcnt left at "no wait").
template <int N>
__device__ __forceinline__ void wait_vm() {
  static_assert(N >= 0 && N < 64, "vmcnt");
  __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (15 << 8) | (((N >> 4) & 3) << 14));
}

// One K stage from an LDS slot. E4M3: each 16x16x128 product is a fresh partial sum that is scaled
// and added into fp32; the products of token tile j+1 are issued before the additions of tile j so the
// matrix core and the vector ALU work side by side.
template <bool FP8, bool GATEUP>
__device__ __forceinline__ void mma_stage(f32x4 (&acc)[4][kTJ], const uint8_t* __restrict__ slot, int wn, int tok0,
                                          int lane) {
  const int tr = lane & 15, g = lane >> 4;
  const uint8_t* A = slot;
  const uint8_t* B = slot + kSlotA;
  const float* SX = reinterpret_cast<const float*>(slot + kSlotS);
  // this wave's four 16-row A tiles: gate/up LDS rows (i < 2 ? 0 : 128) + 32 wn + 16 (i & 1) (gate and
  // up of the same channels); down LDS rows 64 wn + 16 i
  i32x4 a[4][2];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int row = (GATEUP ? (i < 2 ? 0 : 128) + 32 * wn + 16 * (i & 1) : 64 * wn + 16 * i) + tr;
    a[i][0] = *reinterpret_cast<const i32x4*>(A + row * kStageB + ((g ^ (row & 7)) * 16));
    a[i][1] = *reinterpret_cast<const i32x4*>(A + row * kStageB + (((4 + g) ^ (row & 7)) * 16));
  }
  auto load_b = [&](int j, i32x4& b0, i32x4& b1) {
    const int row = tok0 + 16 * j + tr;
    b0 = *reinterpret_cast<const i32x4*>(B + row * kStageB + ((g ^ (row & 7)) * 16));
    b1 = *reinterpret_cast<const i32x4*>(B + row * kStageB + (((4 + g) ^ (row & 7)) * 16));
  };
  if constexpr (FP8) {
    const float s0 = SX[kBM], s1 = SX[kBM + 1];             // weight block scales of this stage
    float swi[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) swi[i] = GATEUP ? (i < 2 ? s0 : s1) : (wn < 2 ? s0 : s1);
    i32x8 aa[4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
      aa[i] = i32x8{a[i][0][0], a[i][0][1], a[i][0][2], a[i][0][3], a[i][1][0], a[i][1][1], a[i][1][2], a[i][1][3]};
    const f32x4 zero = {0.f, 0.f, 0.f, 0.f};
    f32x4 p[2][4];
    float sx[2];
    {
      i32x4 b0, b1;
      load_b(0, b0, b1);
      const i32x8 bb = {b0[0], b0[1], b0[2], b0[3], b1[0], b1[1], b1[2], b1[3]};
#pragma unroll
      for (int i = 0; i < 4; ++i) p[0][i] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(aa[i], bb, zero, 0, 0, 0, 127, 0, 127);
      sx[0] = SX[tok0 + tr];
    }
#pragma unroll
    for (int j = 0; j < kTJ; ++j) {
      const int cur = j & 1, nxt = cur ^ 1;
      if (j + 1 < kTJ) {
        i32x4 b0, b1;
        load_b(j + 1, b0, b1);
        const i32x8 bb = {b0[0], b0[1], b0[2], b0[3], b1[0], b1[1], b1[2], b1[3]};
#pragma unroll
        for (int i = 0; i < 4; ++i)
          p[nxt][i] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(aa[i], bb, zero, 0, 0, 0, 127, 0, 127);
        sx[nxt] = SX[tok0 + 16 * (j + 1) + tr];
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float sc = sx[cur] * swi[i];
#pragma unroll
        for (int r = 0; r < 4; ++r) acc[i][j][r] = fmaf(sc, p[cur][i][r], acc[i][j][r]);
      }
    }
  } else {
#pragma unroll
    for (int j = 0; j < kTJ; ++j) {
      i32x4 b0, b1;
      load_b(j, b0, b1);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a[i][0]),
                                                            __builtin_bit_cast(bf16x8, b0), acc[i][j], 0, 0, 0);
        acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a[i][1]),
                                                            __builtin_bit_cast(bf16x8, b1), acc[i][j], 0, 0, 0);
      }
    }
  }
}

template <bool FP8, bool GATEUP>
__global__ __launch_bounds__(kThreads, 1) void grouped_gemm_mfma(GemmArgs a) {
  extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wn = wave & 3, wm = wave >> 2, tok0 = (128 / kWM) * wm;
  const int esz = FP8 ? 1 : 2;
  const int mt_routed = a.mt_prefix[a.E];
  const int fr = a.f, fs = a.fs;
  const int nt_r = GATEUP ? fr / 128 : a.d / kBW;
  const int nt_s = GATEUP ? fs / 128 : a.d / kBW;
  const int total = mt_routed * nt_r + (fs > 0 ? cdiv(a.T, kBM) * nt_s : 0);

  const int xcd = blockIdx.x & 7, slot_id = blockIdx.x >> 3, per = gridDim.x >> 3;
  const int chunk = cdiv(total, 8);
  const int t_begin = xcd * chunk, t_end = min(total, t_begin + chunk);

  for (int id = t_begin + slot_id; id < t_end; id += per) {
    const TileInfo ti = decode_tile<kBM>(id, a, nt_r, mt_routed);
    const bool shared = ti.group == a.E;
    const int fg = shared ? fs : fr;                       // inner dim of this group
    const int kelems = GATEUP ? a.d : fg;                  // reduction length
    const int kbytes = kelems * esz;
    const int nst = kbytes / kStageB;
    const int kblk = kelems / 128;                         // 128-element scale blocks along K
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

    // ---- loader geometry. Thread tid moves, per stage, A chunks id = q*256 + tid (q < 8) and B chunks
    // id = q*256 + tid (q < 4): LDS row id / 8, LDS position p = id % 8, holding global chunk p ^ (row & 7).
    const int lrow = tid >> 3;                             // row within a kG-row group
    const int lchunk = ((tid & 7) ^ (lrow & 7)) * 16;      // global chunk of this thread's LDS position
    // LDS A row r = kG q + lrow holds weight row c0 + lrow + wrow(q), wrow wave-uniform:
    //   gate/up: rows < 128 are W1 rows c0 + r, rows >= 128 are W3 rows fg + c0 + r - 128;
    //   down:    W2 rows c0 + r.
    const uint8_t* __restrict__ Wl = W + (size_t)(c0 + lrow) * kbytes + lchunk;
    auto wrow_q = [&](int q) -> int {
      const int r0 = kG * q;
      return (GATEUP && r0 >= 128) ? fg + r0 - 128 : r0;
    };
    auto src_row = [&](int r) -> int {
      const int rr = min(r, ti.nrows - 1);
      if (GATEUP) return shared ? ti.rowbase + rr : a.perm_src[ti.rowbase + rr];
      return ti.rowbase + rr;
    };
    uint32_t boff[kBChunks];
#pragma unroll
    for (int q = 0; q < kBChunks; ++q) boff[q] = (uint32_t)src_row(q * kG + lrow) * kbytes + lchunk;
    const uint32_t sxoff = (FP8 && wave < 2) ? (uint32_t)src_row(tid) * kblk : 0u;
    // the tile's two weight block-scale rows: gate/up -> blocks c0/128 (gate) and (fg + c0)/128 (up);
    // down -> blocks c0/128 (row groups 0, 1) and c0/128 + 1 (groups 2, 3). Lanes 0/1 of wave 2 copy them.
    const float* wsrow = FP8 ? WS + (size_t)((lane == 0 ? c0 : (GATEUP ? fg + c0 : c0 + 128)) / 128) * kblk : nullptr;

    auto issue = [&](int kb) {
      uint8_t* slot = lds + (kb % kStages) * kSlot;
      const uint8_t* Xk = X + (size_t)kb * kStageB;
#pragma unroll
      for (int q = 0; q < kAChunks; ++q)
        dma16(Wl + ((size_t)wrow_q(q) * kbytes + (size_t)kb * kStageB), slot + (q * kThreads + wave * 64) * 16);
#pragma unroll
      for (int q = 0; q < kBChunks; ++q) dma16(Xk + boff[q], slot + kSlotA + (q * kThreads + wave * 64) * 16);
      if (FP8 && wave < 2) dma4(XS + sxoff + kb, slot + kSlotS + wave * 256);
      if (FP8 && wave == 2 && lane < 2) dma4(wsrow + kb, slot + kSlotS + kBM * 4);
    };

    f32x4 acc[4][kTJ];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < kTJ; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

    issue(0);
    if (nst > 1) issue(1);
    for (int kb = 0; kb < nst; ++kb) {
      // stage kb landed (stage kb+1 may still be in flight), then every wave is past stage kb-1
      if (kb + 1 < nst) {
        if (FP8 && wave < 3) wait_vm<kAChunks + kBChunks + 1>();
        else wait_vm<kAChunks + kBChunks>();
      } else {
        wait_vm<0>();
      }
      __builtin_amdgcn_s_barrier();
      if (kb + 2 < nst) issue(kb + 2);
      mma_stage<FP8, GATEUP>(acc, lds + (kb % kStages) * kSlot, wn, tok0, lane);
    }
    __builtin_amdgcn_s_barrier();   // every wave is done with the ring before the epilogue reuses it

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
    __syncthreads();   // epilogue LDS reads finish before the next tile's first DMA
  }
}

int gemm_mfma_bm() { return kBM; }

hipError_t launch_gemm_mfma(const GemmArgs& a, bool fp8, bool gateup, int grid, hipStream_t s) {
  static bool attr_done[4] = {false, false, false, false};
  const int k = (fp8 ? 2 : 0) + (gateup ? 1 : 0);
  const void* fn = fp8 ? (gateup ? (const void*)grouped_gemm_mfma<true, true> : (const void*)grouped_gemm_mfma<true, false>)
                       : (gateup ? (const void*)grouped_gemm_mfma<false, true> : (const void*)grouped_gemm_mfma<false, false>);
  if (!attr_done[k]) {
    hipError_t e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, kLdsBytes);
    if (e != hipSuccess) return e;
    attr_done[k] = true;
  }
  if (fp8) {
    if (gateup) grouped_gemm_mfma<true, true><<<grid, kThreads, kLdsBytes, s>>>(a);
    else grouped_gemm_mfma<true, false><<<grid, kThreads, kLdsBytes, s>>>(a);
  } else {
    if (gateup) grouped_gemm_mfma<false, true><<<grid, kThreads, kLdsBytes, s>>>(a);
    else grouped_gemm_mfma<false, false><<<grid, kThreads, kLdsBytes, s>>>(a);
  }
  return hipGetLastError();
}

}  // namespace moe
