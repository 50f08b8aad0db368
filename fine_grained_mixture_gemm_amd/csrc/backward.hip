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

#include <algorithm>

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
// bf16, one 128 x 128 output tile per block (4 waves of 64 x 64). A is the MFMA A operand (output
// columns, so a lane's four accumulators are four adjacent columns of one output row); each
// 16x16x128 product is promoted with the product of its row's and its column's scales. Operands go
// global -> LDS by LDS-DMA into one buffer (16-byte chunks XOR-swizzled by row), three blocks per CU
// overlap each other's waits. Tiles of the shared block (the longest contraction) come first, then the
// routed experts in order; inside a group the larger output dimension runs fastest, so the blocks of
// an XCD (block id mod 8) share the smaller operand and split the larger one.
__global__ __launch_bounds__(256, 3) void grouped_wgrad_mfma(WgGemmArgs a) {
  __shared__ __attribute__((aligned(16))) uint8_t lds[2 * kRowBlk * 128 + 2 * kRowBlk * 4];
  uint8_t* sA = lds;
  uint8_t* sB = lds + kRowBlk * 128;
  float* sAs = reinterpret_cast<float*>(lds + 2 * kRowBlk * 128);
  float* sBs = sAs + kRowBlk;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wn = wave & 1, wm = wave >> 1, tr = lane & 15, g = lane >> 4;
  const int mtn = a.M / 128, ntn = a.N / 128, tpg = mtn * ntn;
  const int t = blockIdx.x;
  const int gi = t / tpg, rem = t - gi * tpg;
  const int group = a.shared ? (gi == 0 ? a.E : gi - 1) : gi;
  int mt, nt;
  if (a.M > a.N) {
    nt = rem / mtn;
    mt = rem - nt * mtn;
  } else {
    mt = rem / ntn;
    nt = rem - mt * ntn;
  }
  const int m0 = mt * 128, n0 = nt * 128;
  const int kb0 = a.pblk[group], nk = a.pblk[group + 1] - kb0;
  // copy geometry: piece 256 q + tid lands at LDS row (256 q + tid) / 8, position tid % 8, which holds
  // global chunk (tid % 8) ^ (row & 7)
  const int prow = tid >> 3, pchunk = ((tid & 7) ^ (prow & 7)) * 16;
  const uint8_t* gA = a.A + (size_t)(n0 + prow) * a.rpad + pchunk;
  const uint8_t* gB = a.B + (size_t)(m0 + prow) * a.rpad + pchunk;
  f32x4 acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
  auto rd = [&](const uint8_t* base, int row) {
    const i32x4 lo = *reinterpret_cast<const i32x4*>(base + row * 128 + ((g ^ (row & 7)) * 16));
    const i32x4 hi = *reinterpret_cast<const i32x4*>(base + row * 128 + (((4 + g) ^ (row & 7)) * 16));
    return i32x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
  };
  for (int s = 0; s < nk; ++s) {
    const size_t kofs = (size_t)(kb0 + s) * kRowBlk;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      dma16(gA + (size_t)(32 * q) * a.rpad + kofs, sA + (q * 256 + wave * 64) * 16);
      dma16(gB + (size_t)(32 * q) * a.rpad + kofs, sB + (q * 256 + wave * 64) * 16);
    }
    if (wave < 2)
      dma4(a.As + (size_t)(kb0 + s) * a.N + n0 + wave * 64 + lane, reinterpret_cast<uint8_t*>(sAs) + wave * 256);
    else
      dma4(a.Bs + (size_t)(kb0 + s) * a.M + m0 + (wave - 2) * 64 + lane, reinterpret_cast<uint8_t*>(sBs) + (wave - 2) * 256);
    wait_vm0();
    barrier_lds();
    i32x8 aa[4];
    f32x4 sa[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      aa[i] = rd(sA, 64 * wn + 16 * i + tr);
      sa[i] = *reinterpret_cast<const f32x4*>(sAs + 64 * wn + 16 * i + 4 * g);
    }
    const f32x4 zero = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const i32x8 bb = rd(sB, 64 * wm + 16 * j + tr);
      const float sb = sBs[64 * wm + 16 * j + tr];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const f32x4 p = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(aa[i], bb, zero, 0, 0, 0, 127, 0, 127);
        acc[i][j] += (sa[i] * sb) * p;
      }
    }
    barrier_lds();   // every wave is done with the buffer before the next stage's copies land in it
  }
  uint16_t* out = (group == a.E ? a.out_s : a.out_r + (size_t)group * a.M * a.N);
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int m = m0 + 64 * wm + 16 * j + tr;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int n = n0 + 64 * wn + 16 * i + 4 * g;
      uint2 v;
      v.x = uint32_t(f32_to_bf16(acc[i][j][0])) | (uint32_t(f32_to_bf16(acc[i][j][1])) << 16);
      v.y = uint32_t(f32_to_bf16(acc[i][j][2])) | (uint32_t(f32_to_bf16(acc[i][j][3])) << 16);
      *reinterpret_cast<uint2*>(out + (size_t)m * a.N + n) = v;
    }
  }
}

int wgrad_row_blocks_max(int T, int K, int E, bool shared) {
  return cdiv(T * K, kRowBlk) + E + (shared ? cdiv(T, kRowBlk) : 0);
}

hipError_t launch_wgrad_prefix(const int32_t* offsets, int E, int T, bool shared, int32_t* pblk, hipStream_t s) {
  wgrad_block_prefix<<<1, 512, 0, s>>>(offsets, E, T, shared ? 1 : 0, pblk);
  return hipGetLastError();
}

hipError_t launch_wgrad_quant(const WgQuantArgs& a, int src, int nblk_max, hipStream_t s) {
  static bool attr_done[4] = {false, false, false, false};
  const void* fns[4] = {(const void*)wgrad_quant_rows<kWgSrcDy>, (const void*)wgrad_quant_rows<kWgSrcX>,
                        (const void*)wgrad_quant_rows<kWgSrcA>, (const void*)wgrad_quant_rows<kWgSrcDgv>};
  if (src < 0 || src > 3) return hipErrorInvalidValue;
  if (nblk_max == 0) return hipSuccess;
  const int ldsb[4] = {wgrad_q_lds<kWgSrcDy>(), wgrad_q_lds<kWgSrcX>(), wgrad_q_lds<kWgSrcA>(), wgrad_q_lds<kWgSrcDgv>()};
  if (!attr_done[src]) {
    const hipError_t e = hipFuncSetAttribute(fns[src], hipFuncAttributeMaxDynamicSharedMemorySize, ldsb[src]);
    if (e != hipSuccess) return e;
    attr_done[src] = true;
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

hipError_t launch_wgrad_gemm(const WgGemmArgs& a, hipStream_t s) {
  const long long tiles = (long long)(a.E + (a.shared ? 1 : 0)) * (a.M / 128) * (a.N / 128);
  if (tiles == 0) return hipSuccess;
  grouped_wgrad_mfma<<<(unsigned)tiles, 256, 0, s>>>(a);
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
