// Input backward of the E4M3 SwiGLU experts: the elementwise part and the weight transposition.
//
// DeepSeek Technical Report: MoE Architecture, 3.6: the activation backward GEMMs run in FP8 with the
// forward's tiling (1x128 activation tiles, 128x128 weight blocks, fp32 promotion every 128). For one
// expert, dx = [dg | dv] [W1; W3] with dg, dv the gradients of a = SiLU(g) * v; the GEMMs are the grouped
// kernels of gemm_mfma.hip (g and v recomputed in fp32; da = dy W2 and dx with the transposed weights).
// A transposed E4M3 weight keeps its codes and takes the transposed grid of its 128x128 block scales.
//
// Weight gradients (same section: the weight backward GEMM in FP8, weight gradients kept in BF16):
// dW2 = dy^T a and d[W1; W3] = [dg | dv]^T x per expert, a contraction over the expert's rows (tokens).
// Both operands are quantized in 1x128 tiles along the rows, starting at the expert's first row (its last
// tile padded with zero rows), and stored transposed so the contraction is contiguous: codes
// [channels][padded rows], scales [row block][channels]. The cached activations x and a enter as the
// values of their forward E4M3 copies (x quantized 1x128 along d, a along f), requantized along the rows.
#include "common.h"
#include "kernels.h"

#include <atomic>

#include <algorithm>
#include <type_traits>
#include <utility>

namespace moe {

// d/dg and d/dv of a = SiLU(g) * v for the upstream da, fp32.
__device__ __forceinline__ void swiglu_grad(float da, float g, float v, float& dg, float& dv) {
  const float sig = 1.0f / (1.0f + __expf(-g));
  dg = da * v * sig * (1.0f + g * (1.0f - sig));
  dv = da * g * sig;
}

// [dg | dv] of a = SiLU(g) * v for the upstream da, evaluated in fp32 and quantized 1x128 (E4M3) along
// the 2 fg columns (dg in columns 0..fg-1, dv in fg..2fg-1). 16 lanes take one (row, 128-column block b):
// lane `sub` holds columns 8 sub .. 8 sub + 7 of block b, for dg and for dv.
//   dv = da * SiLU(g),  dg = da * v * sigmoid(g) * (1 + g * (1 - sigmoid(g)))
__global__ __launch_bounds__(256) void swiglu_backward_quant(const float* __restrict__ da, const float* __restrict__ gv,
                                                             int rows, int fg, uint8_t* __restrict__ q,
                                                             float* __restrict__ scales) {
  const int bpr = fg / 128;
  const long long grp = (long long)blockIdx.x * 16 + (threadIdx.x >> 4);
  if (grp >= (long long)rows * bpr) return;   // 16-lane groups exit together
  const int row = (int)(grp / bpr), b = (int)(grp % bpr), sub = threadIdx.x & 15;
  const size_t c = (size_t)b * 128 + sub * 8;
  const float* dar = da + (size_t)row * fg + c;
  const float* gr = gv + (size_t)row * 2 * fg + c;
  float d8[8], g8[8], v8[8];
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const float4 x = *reinterpret_cast<const float4*>(dar + 4 * h);
    const float4 y = *reinterpret_cast<const float4*>(gr + 4 * h);
    const float4 z = *reinterpret_cast<const float4*>(gr + fg + 4 * h);
    d8[4 * h] = x.x; d8[4 * h + 1] = x.y; d8[4 * h + 2] = x.z; d8[4 * h + 3] = x.w;
    g8[4 * h] = y.x; g8[4 * h + 1] = y.y; g8[4 * h + 2] = y.z; g8[4 * h + 3] = y.w;
    v8[4 * h] = z.x; v8[4 * h + 1] = z.y; v8[4 * h + 2] = z.z; v8[4 * h + 3] = z.w;
  }
  float dg[8], dv[8], mg = 0.f, mv = 0.f;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    swiglu_grad(d8[i], g8[i], v8[i], dg[i], dv[i]);
    mg = fmaxf(mg, fabsf(dg[i]));
    mv = fmaxf(mv, fabsf(dv[i]));
  }
#pragma unroll
  for (int o = 8; o > 0; o >>= 1) {
    mg = fmaxf(mg, __shfl_xor(mg, o, 64));
    mv = fmaxf(mv, __shfl_xor(mv, o, 64));
  }
  float sg, ig, sv, iv;
  e4m3_scales(mg, sg, ig);
  e4m3_scales(mv, sv, iv);
  uint8_t* qr = q + (size_t)row * 2 * fg + c;
  uint2 og, ov;
  og.x = f32x4_to_e4m3x4(dg[0] * ig, dg[1] * ig, dg[2] * ig, dg[3] * ig);
  og.y = f32x4_to_e4m3x4(dg[4] * ig, dg[5] * ig, dg[6] * ig, dg[7] * ig);
  ov.x = f32x4_to_e4m3x4(dv[0] * iv, dv[1] * iv, dv[2] * iv, dv[3] * iv);
  ov.y = f32x4_to_e4m3x4(dv[4] * iv, dv[5] * iv, dv[6] * iv, dv[7] * iv);
  *reinterpret_cast<uint2*>(qr) = og;
  *reinterpret_cast<uint2*>(qr + fg) = ov;
  if (sub == 0) {
    scales[(size_t)row * 2 * bpr + b] = sg;
    scales[(size_t)row * 2 * bpr + bpr + b] = sv;
  }
}

// qt[m][c][r] = q[m][r][c] for a batch of byte matrices [rows, cols] (multiples of 64), 64 x 64 tiles
// through LDS: each thread reads 16 bytes of a row and writes 16 bytes of a column.
__global__ __launch_bounds__(256) void transpose_u8(const uint8_t* __restrict__ q, int rows, int cols,
                                                    uint8_t* __restrict__ qt) {
  __shared__ __attribute__((aligned(16))) uint8_t tile[64][80];
  const int c0 = blockIdx.x * 64, r0 = blockIdx.y * 64;
  const size_t mat = (size_t)blockIdx.z * rows * cols;
  const int t = threadIdx.x, lr = t >> 2, lc = (t & 3) * 16;
  *reinterpret_cast<uint4*>(&tile[lr][lc]) = *reinterpret_cast<const uint4*>(q + mat + (size_t)(r0 + lr) * cols + c0 + lc);
  __syncthreads();
  uint8_t b[16];
#pragma unroll
  for (int k = 0; k < 16; ++k) b[k] = tile[lc + k][lr];
  uint4 o;
  o.x = b[0] | (b[1] << 8) | (b[2] << 16) | ((uint32_t)b[3] << 24);
  o.y = b[4] | (b[5] << 8) | (b[6] << 16) | ((uint32_t)b[7] << 24);
  o.z = b[8] | (b[9] << 8) | (b[10] << 16) | ((uint32_t)b[11] << 24);
  o.w = b[12] | (b[13] << 8) | (b[14] << 16) | ((uint32_t)b[15] << 24);
  *reinterpret_cast<uint4*>(qt + mat + (size_t)(c0 + lr) * rows + r0 + lc) = o;
}

// st[m][c][r] = s[m][r][c] for a batch of small fp32 matrices [rb, cb].
__global__ __launch_bounds__(256) void transpose_f32(const float* __restrict__ s, long long batch, int rb, int cb,
                                                     float* __restrict__ st) {
  const long long n = batch * rb * cb;
  for (long long i = (long long)blockIdx.x * 256 + threadIdx.x; i < n; i += (long long)gridDim.x * 256) {
    const long long m = i / ((long long)rb * cb);
    const int rem = (int)(i - m * rb * cb), r = rem / cb, c = rem % cb;
    st[m * rb * cb + (long long)c * rb + r] = s[i];
  }
}

// ----------------------------------------------------------------------------- weight gradients
constexpr int kRowBlk = 128;                       // rows per quantization tile = rows per GEMM K stage
// Staging of a row block in LDS, as narrow as the values allow (more blocks per CU in flight): [dg | dv]
// fp32; dy its bf16 bits; x and a their forward E4M3 codes plus one scale per row (the dequantized value
// code * scale is formed again when read, the same fp32 product). Then an LDS copy of pblk (E <= 256).
// [dg | dv] blocks take 32 channels of f and produce their 32 dg and 32 dv columns from one read of da,
// g and v (64 output channels); the others take 128 channels (x and a are first quantized along 128
// channels per row).
template <int SRC>
constexpr int wgrad_q_elem() { return SRC == kWgSrcDgv ? 4 : SRC == kWgSrcDy ? 2 : 1; }
template <int SRC>
constexpr int wgrad_q_cw() { return SRC == kWgSrcDgv ? 64 : 128; }
template <int SRC>
constexpr int wgrad_q_stride() { return wgrad_q_cw<SRC>() + 1; }   // odd: column reads spread over the banks
template <int SRC>
constexpr int wgrad_q_lds() {
  return (kRowBlk * wgrad_q_stride<SRC>() * wgrad_q_elem<SRC>() + 3) / 4 * 4 + kRowBlk * 4 + 258 * 4;
}

// pblk[g] = first row block of group g (routed experts 0..E-1, then the shared block, empty unless
// `shared`), pblk[E + 1] = their total: ceil(n_g / 128) blocks per group. One block, a scan over LDS.
// pblk[E + 2 .. E + 19] are cleared: the tile counters of the two weight-gradient GEMMs.
__global__ __launch_bounds__(512) void wgrad_block_prefix(const int32_t* __restrict__ offsets, int E, int T,
                                                          int shared, int32_t* __restrict__ pblk) {
  __shared__ int buf[512];
  const int g = threadIdx.x;
  int n = 0;
  if (g < E) n = cdiv(offsets[g + 1] - offsets[g], kRowBlk);
  else if (g == E && shared) n = cdiv(T, kRowBlk);
  buf[g] = n;
  __syncthreads();
  for (int o = 1; o < 512; o <<= 1) {
    const int v = g >= o ? buf[g - o] : 0;
    __syncthreads();
    buf[g] += v;
    __syncthreads();
  }
  if (g <= E) pblk[g + 1] = buf[g];
  if (g == 0) pblk[0] = 0;
  if (g < 18) pblk[E + 2 + g] = 0;   // the weight-gradient GEMMs' tile counters (9 per launch)
}

// The group holding row block b: the last g with pblk[g] <= b (a non-empty group; b < pblk[E + 1]).
__device__ __forceinline__ int wgrad_group_of(const int32_t* __restrict__ pblk, int E, int b) {
  int lo = 0, hi = E + 1;
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (pblk[mid] <= b) lo = mid;
    else hi = mid;
  }
  return lo;
}

// One block per (row block b, channel block): the block's rows are staged in LDS (source dependent,
// below), then every channel is quantized over the 128 rows and written transposed.
//   DY : dy rows (bf16) as given;
//   X  : u rows (bf16, routed rows gathered through perm) -> 1x128 E4M3 along the channels, as the
//        forward quantizes them, dequantized;
//   A  : a = SiLU(g) * v from the fp32 [g | v] rows -> the forward's 1x128 requantization, dequantized;
//   DGV: dg and dv of 32 channels of f from da and [g | v], fp32 (output channels c and fg + c).
template <int SRC>
__global__ __launch_bounds__(256) void wgrad_quant_rows(WgQuantArgs a) {
  extern __shared__ __attribute__((aligned(16))) uint8_t qlds[];
  constexpr int kCW = wgrad_q_cw<SRC>(), kS = wgrad_q_stride<SRC>();
  constexpr int kLPR = SRC == kWgSrcDgv ? 4 : kCW / 8, kRPP = 256 / kLPR;   // lanes per row, rows per pass
  constexpr int kTileB = (kRowBlk * kS * wgrad_q_elem<SRC>() + 3) / 4 * 4;
  float* rs = reinterpret_cast<float*>(qlds + kTileB);            // row scales (x, a)
  int32_t* pb = reinterpret_cast<int32_t*>(qlds + kTileB + kRowBlk * 4);
  const int b = blockIdx.x, cb = blockIdx.y, tid = threadIdx.x;
  if (b >= a.pblk[a.E + 1]) return;
  // the group search runs on an LDS copy of the prefix (a search over global memory would wait for nine
  // dependent loads)
  for (int i = tid; i <= a.E + 1; i += 256) pb[i] = a.pblk[i];
  __syncthreads();
  const int grp = wgrad_group_of(pb, a.E, b);
  const bool shared = grp == a.E;
  const int r0 = (b - pb[grp]) * kRowBlk;
  const int n = shared ? a.T : a.offsets[grp + 1] - a.offsets[grp];
  const int nrows = min(kRowBlk, n - r0);
  const int rowbase = (shared ? 0 : a.offsets[grp]) + r0;
  const int c8 = (tid % kLPR) * 8;
#pragma unroll 4
  for (int pass = 0; pass < kRowBlk / kRPP; ++pass) {
    const int rr = pass * kRPP + tid / kLPR;
    float v[8];
    if (rr < nrows) {                              // uniform over the lanes of a row
      const int row = rowbase + rr;
      if constexpr (SRC == kWgSrcDy || SRC == kWgSrcX) {
        const uint16_t* base = shared ? a.bf_s : a.bf_r;
        const size_t srow = SRC == kWgSrcX && !shared ? (size_t)a.perm[row] : (size_t)row;
        const uint4 raw = *reinterpret_cast<const uint4*>(base + srow * a.C + cb * kCW + c8);
        const uint32_t w[4] = {raw.x, raw.y, raw.z, raw.w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          v[2 * i] = __uint_as_float(w[i] << 16);
          v[2 * i + 1] = __uint_as_float(w[i] & 0xFFFF0000u);
        }
      } else if constexpr (SRC == kWgSrcA) {
        const float* gr = (shared ? a.gv_s : a.gv_r) + (size_t)row * 2 * a.fg + cb * kCW + c8;
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          const float4 g4 = *reinterpret_cast<const float4*>(gr + 4 * h);
          const float4 v4 = *reinterpret_cast<const float4*>(gr + a.fg + 4 * h);
          v[4 * h] = silu(g4.x) * v4.x;
          v[4 * h + 1] = silu(g4.y) * v4.y;
          v[4 * h + 2] = silu(g4.z) * v4.z;
          v[4 * h + 3] = silu(g4.w) * v4.w;
        }
      } else {
        const int c = cb * 32 + c8;
        const float* gr = (shared ? a.gv_s : a.gv_r) + (size_t)row * 2 * a.fg + c;
        const float* dr = (shared ? a.da_s : a.da_r) + (size_t)row * a.fg + c;
        float d8[8], g8[8], u8[8];
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          const float4 x = *reinterpret_cast<const float4*>(dr + 4 * h);
          const float4 y = *reinterpret_cast<const float4*>(gr + 4 * h);
          const float4 z = *reinterpret_cast<const float4*>(gr + a.fg + 4 * h);
          d8[4 * h] = x.x; d8[4 * h + 1] = x.y; d8[4 * h + 2] = x.z; d8[4 * h + 3] = x.w;
          g8[4 * h] = y.x; g8[4 * h + 1] = y.y; g8[4 * h + 2] = y.z; g8[4 * h + 3] = y.w;
          u8[4 * h] = z.x; u8[4 * h + 1] = z.y; u8[4 * h + 2] = z.z; u8[4 * h + 3] = z.w;
        }
        float* t = reinterpret_cast<float*>(qlds) + rr * kS + c8;
#pragma unroll
        for (int k = 0; k < 8; ++k) {
          float dg, dv;
          swiglu_grad(d8[k], g8[k], u8[k], dg, dv);
          t[k] = dg;
          t[32 + k] = dv;
        }
      }
      if constexpr (SRC == kWgSrcX || SRC == kWgSrcA) {
        float amax = 0.f;
#pragma unroll
        for (int k = 0; k < 8; ++k) amax = fmaxf(amax, fabsf(v[k]));
#pragma unroll
        for (int o = 8; o > 0; o >>= 1) amax = fmaxf(amax, __shfl_xor(amax, o, 64));
        float sc, inv;
        e4m3_scales(amax, sc, inv);
        const uint32_t q0 = f32x4_to_e4m3x4(v[0] * inv, v[1] * inv, v[2] * inv, v[3] * inv);
        const uint32_t q1 = f32x4_to_e4m3x4(v[4] * inv, v[5] * inv, v[6] * inv, v[7] * inv);
        uint8_t* t8 = qlds + rr * kS + c8;
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          t8[k] = uint8_t(q0 >> (8 * k));
          t8[4 + k] = uint8_t(q1 >> (8 * k));
        }
        if ((tid & 15) == 0) rs[rr] = sc;
      } else if constexpr (SRC == kWgSrcDy) {
        uint16_t* t16 = reinterpret_cast<uint16_t*>(qlds) + rr * kS + c8;
#pragma unroll
        for (int k = 0; k < 8; ++k) t16[k] = uint16_t(__float_as_uint(v[k]) >> 16);
      }
    } else {
      // rows past the group's end are zero
      if constexpr (SRC == kWgSrcX || SRC == kWgSrcA) {
        uint8_t* t8 = qlds + rr * kS + c8;
#pragma unroll
        for (int k = 0; k < 8; ++k) t8[k] = 0;
        if ((tid & 15) == 0) rs[rr] = 0.f;
      } else if constexpr (SRC == kWgSrcDy) {
        uint16_t* t16 = reinterpret_cast<uint16_t*>(qlds) + rr * kS + c8;
#pragma unroll
        for (int k = 0; k < 8; ++k) t16[k] = 0;
      } else {
        float* t = reinterpret_cast<float*>(qlds) + rr * kS + c8;
#pragma unroll
        for (int k = 0; k < 8; ++k) t[k] = t[32 + k] = 0.f;
      }
    }
  }
  __syncthreads();
  // 8 lanes per channel, 16 consecutive rows each: one store instruction of a wave writes the whole
  // 128-row run of 8 channels (8 full cache lines of the transposed output)
  const int lane = tid & 63, wave = tid >> 6, sub = lane & 7, cl = lane >> 3;
#pragma unroll 1
  for (int pass = 0; pass < kCW / 32; ++pass) {
    const int c = pass * 32 + wave * 8 + cl;
    float v[16];
    float amax = 0.f;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int row = 16 * sub + r;
      if constexpr (SRC == kWgSrcX || SRC == kWgSrcA)
        v[r] = __builtin_amdgcn_cvt_f32_fp8((int)qlds[row * kS + c], 0) * rs[row];
      else if constexpr (SRC == kWgSrcDy)
        v[r] = __uint_as_float(uint32_t(reinterpret_cast<const uint16_t*>(qlds)[row * kS + c]) << 16);
      else
        v[r] = reinterpret_cast<const float*>(qlds)[row * kS + c];
      amax = fmaxf(amax, fabsf(v[r]));
    }
    amax = fmaxf(amax, __shfl_xor(amax, 1, 64));
    amax = fmaxf(amax, __shfl_xor(amax, 2, 64));
    amax = fmaxf(amax, __shfl_xor(amax, 4, 64));
    float sc, inv;
    e4m3_scales(amax, sc, inv);
    uint32_t o[4];
#pragma unroll
    for (int k = 0; k < 4; ++k)
      o[k] = f32x4_to_e4m3x4(v[4 * k] * inv, v[4 * k + 1] * inv, v[4 * k + 2] * inv, v[4 * k + 3] * inv);
    const int gc = SRC == kWgSrcDgv ? (c < 32 ? cb * 32 + c : a.fg + cb * 32 + c - 32) : cb * kCW + c;
    *reinterpret_cast<uint4*>(a.qt + (size_t)gc * a.rpad + (size_t)b * kRowBlk + 16 * sub) = uint4{o[0], o[1], o[2], o[3]};
    if (sub == 0) a.st[(size_t)b * a.C + gc] = sc;
  }
}

// out[m][n] = sum over the group's row blocks kb of  sum_{k in kb} B[m][k] A[n][k] * sB[kb][m] sA[kb][n],
// bf16. One persistent block of 512 threads (8 waves, two per SIMD) per CU takes 256 x 256 output tiles;
// the K dimension of a tile is its group's row blocks (128 rows = one 16x16x128 MFMA deep, promoted into
// fp32 with the product of its row's and its column's scales). Both operands go global -> LDS by LDS-DMA
// into a ring of two stages (16-byte chunks XOR-swizzled by row); the loader runs one stage ahead, also
// across tile boundaries. Wave w multiplies output columns 64 (w mod 4).. and rows 128 (w div 4)..: A is
// the MFMA A operand, so a lane's accumulators are output columns. The A rows of a stage are loaded in the
// column order that gives each lane 8 adjacent columns of one output row per pair of 16-column MFMA
// tiles, and a tile's bf16 result is stored during the next tile's first stage (its stores then complete
// behind that stage's MFMAs). Tile list: the shared block first (the longest contraction), then the
// routed experts; inside a group the output rows run fastest. The first 7/8 of the list's estimated cost
// (stages + 1 per tile) is cut into eight ranges, one per XCD (block id mod 8), whose blocks take tiles in
// order from the XCD's counter and then from the pool of the remaining tiles. A tile of an empty group
// multiplies nothing and stores zeros.
constexpr int kWgT = 256;
constexpr int kWgThreads = 512;
constexpr int kWgOp = kWgT * 128;                  // one operand of a stage: 256 rows x 128 bytes
constexpr int kWgSlot = 2 * kWgOp + 2 * kWgT * 4;  // both operands + their scales
constexpr int kWgIds = 2 * kWgSlot;                // ring of the block's next tile ids
constexpr int kWgLds = kWgIds + 16;
static_assert(kWgLds <= 160 * 1024, "LDS");

// Output column (within a wave's 64) of A row l = 16 i + 4 g + r of the stage: a lane of group g holds, for
// MFMA tiles 2p and 2p + 1, columns 32 p + 8 g + 0..7.
__device__ __forceinline__ int wgrad_col_of(int l) {
  const int i = l >> 4, g = (l >> 2) & 3, r = l & 3;
  return 32 * (i >> 1) + 8 * g + 4 * (i & 1) + r;
}

__global__ __launch_bounds__(kWgThreads, 1) void grouped_wgrad_mfma(WgGemmArgs a) {
  extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wn = wave & 3, wm = wave >> 2, tr = lane & 15, g = lane >> 4;
  const int E = a.E, M = a.M, N = a.N;
  const bool has_shared = a.shared != 0;
  const int G = E + (has_shared ? 1 : 0);
  const int mtn = (M + kWgT - 1) / kWgT, ntn = (N + kWgT - 1) / kWgT, tpg = mtn * ntn;
  const int32_t* pb = a.pblk;
  const int S = pb[E + 1];
  const int nks = has_shared ? S - pb[E] : 0;
  // row blocks of the groups before position go of the tile list, and the group at that position
  auto stages_before = [&](int go) { return has_shared ? (go == 0 ? 0 : nks + pb[go - 1]) : pb[go]; };
  auto group_at = [&](int go) { return has_shared ? (go == 0 ? E : go - 1) : go; };
  // first tile of XCD x's range: cost of the tiles before tile go * tpg + r is tpg (stages_before(go) + go)
  // + r (stages of group go + 1)
  // the eight XCD ranges cover the first 7/8 of the cost; the tiles after them are a pool (counter 8)
  auto range_start = [&](int x) {
    if (x >= 9) return G * tpg;
    const long long ranged = (long long)tpg * (S + G) - (long long)tpg * (S + G) / 8;
    const long long target = ranged * x / 8;
    int lo = 0, hi = G;
    while (hi - lo > 1) {
      const int mid = (lo + hi) >> 1;
      if ((long long)tpg * (stages_before(mid) + mid) <= target) lo = mid;
      else hi = mid;
    }
    const long long rem = target - (long long)tpg * (stages_before(lo) + lo);
    const int c = stages_before(lo + 1) - stages_before(lo) + 1;
    return lo * tpg + (int)min((rem + c - 1) / c, (long long)tpg);
  };
  const int xcd = blockIdx.x & 7;
  const int t_begin = range_start(xcd), t_end = range_start(xcd + 1);
  const int p_begin = range_start(8), n_tiles = G * tpg;
  // the next tile id: from this XCD's range, then from the pool; n_tiles: none left
  auto claim = [&]() {
    const int id = t_begin + atomicAdd(a.xcount + xcd, 1);
    if (id < t_end) return id;
    const int p = p_begin + atomicAdd(a.xcount + 8, 1);
    return p < n_tiles ? p : n_tiles;
  };
  int32_t* ids = reinterpret_cast<int32_t*>(lds + kWgIds);
  int pending = 0;
  if (tid == 0) {
#pragma unroll
    for (int k = 0; k < 3; ++k) ids[k] = claim();
    pending = claim();
  }
  barrier_lds();
  int id_l = __builtin_amdgcn_readfirstlane(ids[0]);
  if (id_l >= n_tiles) return;
  int ktile = 0;

  // ---- loader. Thread tid moves, per stage and operand, the 16-byte pieces 512 q + tid (q < 4): LDS row
  // 64 q + lrow, position tid % 8, which holds global chunk (tid % 8) ^ (lrow % 8). LDS A row 64 q + l is
  // output column 64 q + wgrad_col_of(l) of the tile.
  const int lrow = tid >> 3;
  const int lchunk = ((tid & 7) ^ (lrow & 7)) * 16;
  const int acol = wgrad_col_of(lrow);
  struct Tile {
    int group, m0, n0, kb0, nk;
  };
  auto decode = [&](int id) {
    Tile t;
    const int go = id / tpg, rem = id - go * tpg;
    t.group = group_at(go);
    const int nt = rem / mtn;
    t.m0 = (rem - nt * mtn) * kWgT;
    t.n0 = nt * kWgT;
    t.kb0 = pb[t.group];
    t.nk = pb[t.group + 1] - t.kb0;
    return t;
  };
  Tile tl = decode(id_l);
  // per tile: this thread's A and B row pointers for q = 0 (rows q = 1..3 follow at 64-row steps; in a tile
  // that ends 128 rows early, rows past the end re-read the valid half) and its wave's scale pointer
  const uint8_t* pA = nullptr;
  const uint8_t* pB = nullptr;
  const float* ps = nullptr;
  int kl = 0, started = 1, nst_l = 1, a_half = 0, b_half = 0;
  bool live = true;
  auto setup = [&]() {
    // an empty group re-reads row block 0 (never multiplied): its own start may lie past the last block
    const int kb0 = tl.nk > 0 ? tl.kb0 : 0;
    nst_l = max(tl.nk, 1);
    a_half = tl.n0 + kWgT > N ? 2 : 4;   // q >= a_half: rows past the end
    b_half = tl.m0 + kWgT > M ? 2 : 4;
    pA = a.A + (size_t)(tl.n0 + acol) * a.rpad + (size_t)kb0 * 128 + lchunk;
    pB = a.B + (size_t)(tl.m0 + lrow) * a.rpad + (size_t)kb0 * 128 + lchunk;
    if (wave < 4) {
      const int q = wave < a_half ? wave : wave - 2;
      ps = a.As + (size_t)kb0 * N + tl.n0 + 64 * q + wgrad_col_of(lane);
    } else {
      // B scale position 128 h + 8 t + j holds row 128 h + 16 j + t: a lane reads its eight in one go
      const int h = wave - 4 < b_half ? (wave - 4) >> 1 : 0;
      const int pos = ((wave - 4) & 1) * 64 + lane;
      ps = a.Bs + (size_t)kb0 * M + tl.m0 + 128 * h + 16 * (pos & 7) + (pos >> 3);
    }
    kl = 0;
  };
  setup();
  auto issue = [&](uint8_t* sl) {
    if (kl == nst_l && live) {
      ++ktile;
      id_l = __builtin_amdgcn_readfirstlane(ids[ktile & 3]);
      if (id_l < n_tiles) {
        tl = decode(id_l);
        setup();
        ++started;
        // the id of tile ktile + 2 arrived a tile ago; request the one after it
        if (tid == 0) {
          ids[(ktile + 2) & 3] = pending;
          pending = claim();
        }
      } else {
        live = false;
      }
    }
    const size_t kofs = (size_t)(live ? kl : 0) * 128;
    ++kl;
#pragma unroll
    for (int q = 0; q < 4; ++q)
      dma16(pA + (size_t)(64 * (q < a_half ? q : q - 2)) * a.rpad + kofs, sl + (q * kWgThreads + wave * 64) * 16);
#pragma unroll
    for (int q = 0; q < 4; ++q)
      dma16(pB + (size_t)(64 * (q < b_half ? q : q - 2)) * a.rpad + kofs, sl + kWgOp + (q * kWgThreads + wave * 64) * 16);
    dma4(ps + (kofs / 128) * (wave < 4 ? N : M), sl + 2 * kWgOp + wave * 256);
  };

  auto rd = [&](const uint8_t* base, int row) {
    const i32x4 lo = *reinterpret_cast<const i32x4*>(base + row * 128 + ((g ^ (row & 7)) * 16));
    const i32x4 hi = *reinterpret_cast<const i32x4*>(base + row * 128 + (((4 + g) ^ (row & 7)) * 16));
    return i32x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
  };

  // ---- compute: the tile being multiplied, and the bf16 result of the previous one awaiting its stores
  Tile tc = tl;
  int nst_c = nst_l, done = 0;
  f32x4 acc[4][8];
  uint4 res[8][2];
  uint16_t* res_out = nullptr;   // this lane's first output of the pending result; null: nothing to store
  // One stage: wait for its copies, start the next stage's, store the pending result (first stage of a
  // tile), multiply. FIRST: the products initialise the accumulators.
  auto stage = [&](int gs, auto first_tag) {
    constexpr bool FIRST = decltype(first_tag)::value;
    uint8_t* cur = lds + (gs & 1) * kWgSlot;
    wait_vm0();       // this wave's copies of stage gs (and the previous stores) are done
    barrier_lds();    // ... and every wave's; every wave is done with the other slot
    issue(lds + ((gs + 1) & 1) * kWgSlot);
    if constexpr (FIRST) {
      if (res_out) {
#pragma unroll
        for (int j = 0; j < 8; ++j)
#pragma unroll
          for (int p = 0; p < 2; ++p) *reinterpret_cast<uint4*>(res_out + (size_t)(16 * j) * N + 32 * p) = res[j][p];
      }
    }
    const bool active = tc.nk > 0 && tc.n0 + 64 * wn < N && tc.m0 + 128 * wm < M;
    if (active) {
      const uint8_t* sA = cur;
      const uint8_t* sB = cur + kWgOp;
      const float* sAs = reinterpret_cast<const float*>(cur + 2 * kWgOp);
      const float* sBs = sAs + kWgT;
      i32x8 aa[4];
      f32x4 sa[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        aa[i] = rd(sA, 64 * wn + 16 * i + tr);
        sa[i] = *reinterpret_cast<const f32x4*>(sAs + 64 * wn + 16 * i + 4 * g);
      }
      // the B rows and scales of the next 16-row tile load while the current one multiplies; each product
      // is promoted one MFMA after it is issued, so the matrix core and the vector ALU overlap
      i32x8 bb[2];
      const f32x4 sb0 = *reinterpret_cast<const f32x4*>(sBs + 128 * wm + 8 * tr);
      const f32x4 sb1 = *reinterpret_cast<const f32x4*>(sBs + 128 * wm + 8 * tr + 4);
      const float sbv[8] = {sb0[0], sb0[1], sb0[2], sb0[3], sb1[0], sb1[1], sb1[2], sb1[3]};
      bb[0] = rd(sB, 128 * wm + tr);
      const f32x4 zero = {0.f, 0.f, 0.f, 0.f};
      f32x4 pr[2], cs[4];
      auto promote = [&](int i, int j, const f32x4& p, const f32x4& c) {
        if constexpr (FIRST) acc[i][j] = c * p;
        else acc[i][j] += c * p;
      };
      [&]<int... J>(std::integer_sequence<int, J...>) {
        ([&] {
          constexpr int j = J;
          if constexpr (j + 1 < 8) bb[(j + 1) & 1] = rd(sB, 128 * wm + 16 * (j + 1) + tr);
          [&]<int... I>(std::integer_sequence<int, I...>) {
            ([&] {
              constexpr int i = I;
              pr[i & 1] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(aa[i], bb[j & 1], zero, 0, 0, 0, 127, 0, 127);
              if constexpr (i > 0) promote(i - 1, j, pr[(i - 1) & 1], cs[i - 1]);
              else if constexpr (j > 0) promote(3, j - 1, pr[1], cs[3]);
              cs[i] = sa[i] * sbv[j];
            }(), ...);
          }(std::make_integer_sequence<int, 4>{});
        }(), ...);
      }(std::make_integer_sequence<int, 8>{});
      promote(3, 7, pr[1], cs[3]);
    } else if constexpr (FIRST) {
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 8; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
    }
  };

  issue(lds);
  for (int gs = 0;;) {
    stage(gs++, std::true_type{});
    for (int kb = 1; kb < nst_c; ++kb) stage(gs++, std::false_type{});

    // ---- tile tc is complete: lane holds, for output row m0 + 128 wm + 16 j + tr, columns
    // n0 + 64 wn + 32 p + 8 g + 0..7 in acc[2p][j], acc[2p + 1][j]
    const bool valid = tc.n0 + 64 * wn < N && tc.m0 + 128 * wm < M;
    uint16_t* out = tc.group == E ? a.out_s : a.out_r + (size_t)tc.group * M * N;
    res_out = valid ? out + (size_t)(tc.m0 + 128 * wm + tr) * N + tc.n0 + 64 * wn + 8 * g : nullptr;
#pragma unroll
    for (int j = 0; j < 8; ++j)
#pragma unroll
      for (int p = 0; p < 2; ++p) {
        const f32x4 x = acc[2 * p][j], y = acc[2 * p + 1][j];
        res[j][p] = uint4{uint32_t(f32_to_bf16(x[0])) | (uint32_t(f32_to_bf16(x[1])) << 16),
                          uint32_t(f32_to_bf16(x[2])) | (uint32_t(f32_to_bf16(x[3])) << 16),
                          uint32_t(f32_to_bf16(y[0])) | (uint32_t(f32_to_bf16(y[1])) << 16),
                          uint32_t(f32_to_bf16(y[2])) | (uint32_t(f32_to_bf16(y[3])) << 16)};
      }
    if (++done == started && !live) break;
    // the loader moved to this tile while the last stage of the previous one was multiplied
    tc = tl;
    nst_c = nst_l;
  }
  if (res_out) {
#pragma unroll
    for (int j = 0; j < 8; ++j)
#pragma unroll
      for (int p = 0; p < 2; ++p) *reinterpret_cast<uint4*>(res_out + (size_t)(16 * j) * N + 32 * p) = res[j][p];
  }
  wait_vm0();
}

int wgrad_row_blocks_max(int T, int K, int E, bool shared) {
  return cdiv(T * K, kRowBlk) + E + (shared ? cdiv(T, kRowBlk) : 0);
}

hipError_t launch_wgrad_prefix(const int32_t* offsets, int E, int T, bool shared, int32_t* pblk, hipStream_t s) {
  wgrad_block_prefix<<<1, 512, 0, s>>>(offsets, E, T, shared ? 1 : 0, pblk);
  return hipGetLastError();
}

hipError_t launch_wgrad_quant(const WgQuantArgs& a, int src, int nblk_max, hipStream_t s) {
  static std::atomic<bool> attr_done[4];   // set once per kernel (setting it twice is harmless)
  const void* fns[4] = {(const void*)wgrad_quant_rows<kWgSrcDy>, (const void*)wgrad_quant_rows<kWgSrcX>,
                        (const void*)wgrad_quant_rows<kWgSrcA>, (const void*)wgrad_quant_rows<kWgSrcDgv>};
  if (src < 0 || src > 3) return hipErrorInvalidValue;
  if (nblk_max == 0) return hipSuccess;
  const int ldsb[4] = {wgrad_q_lds<kWgSrcDy>(), wgrad_q_lds<kWgSrcX>(), wgrad_q_lds<kWgSrcA>(), wgrad_q_lds<kWgSrcDgv>()};
  if (!attr_done[src].load(std::memory_order_relaxed)) {
    const hipError_t e = hipFuncSetAttribute(fns[src], hipFuncAttributeMaxDynamicSharedMemorySize, ldsb[src]);
    if (e != hipSuccess) return e;
    attr_done[src].store(true, std::memory_order_relaxed);
  }
  const dim3 grid(nblk_max, a.C / 128), grid64(nblk_max, a.C / 64);
  switch (src) {
    case kWgSrcDy: wgrad_quant_rows<kWgSrcDy><<<grid, 256, ldsb[0], s>>>(a); break;
    case kWgSrcX: wgrad_quant_rows<kWgSrcX><<<grid, 256, ldsb[1], s>>>(a); break;
    case kWgSrcA: wgrad_quant_rows<kWgSrcA><<<grid, 256, ldsb[2], s>>>(a); break;
    default: wgrad_quant_rows<kWgSrcDgv><<<grid64, 256, ldsb[3], s>>>(a); break;
  }
  return hipGetLastError();
}

hipError_t launch_wgrad_gemm(const WgGemmArgs& a, int grid, hipStream_t s) {
  static std::atomic<bool> attr_done{false};   // set once (setting it twice is harmless)
  if (!attr_done.load(std::memory_order_relaxed)) {
    const hipError_t e = hipFuncSetAttribute((const void*)grouped_wgrad_mfma, hipFuncAttributeMaxDynamicSharedMemorySize, kWgLds);
    if (e != hipSuccess) return e;
    attr_done.store(true, std::memory_order_relaxed);
  }
  grouped_wgrad_mfma<<<grid, kWgThreads, kWgLds, s>>>(a);
  return hipGetLastError();
}

hipError_t launch_swiglu_backward_quant(const float* da, const float* gv, int rows, int fg, uint8_t* q, float* scales,
                                        hipStream_t s) {
  const long long groups = (long long)rows * (fg / 128);
  if (groups == 0) return hipSuccess;
  swiglu_backward_quant<<<(unsigned)((groups + 15) / 16), 256, 0, s>>>(da, gv, rows, fg, q, scales);
  return hipGetLastError();
}

hipError_t launch_transpose_fp8(const uint8_t* q, const float* scales, int batch, int rows, int cols, uint8_t* qt,
                                float* scales_t, hipStream_t s) {
  if (batch == 0) return hipSuccess;
  transpose_u8<<<dim3(cols / 64, rows / 64, batch), 256, 0, s>>>(q, rows, cols, qt);
  const long long n = (long long)batch * (rows / 128) * (cols / 128);
  transpose_f32<<<(unsigned)std::min<long long>((n + 255) / 256, 4096), 256, 0, s>>>(scales, batch, rows / 128,
                                                                                    cols / 128, scales_t);
  return hipGetLastError();
}

}  // namespace moe
