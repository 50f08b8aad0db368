// Input backward of the E4M3 SwiGLU experts: the elementwise part and the weight transposition.
//
// DeepSeek Technical Report: MoE Architecture, 3.6: the activation backward GEMMs run in FP8 with the
// forward's tiling (1x128 activation tiles, 128x128 weight blocks, fp32 promotion every 128). For one
// expert, dx = [dg | dv] [W1; W3] with dg, dv the gradients of a = SiLU(g) * v; the GEMMs are the grouped
// kernels of gemm_mfma.hip (g and v recomputed in fp32; da = dy W2 and dx with the transposed weights).
// A transposed E4M3 weight keeps its codes and takes the transposed grid of its 128x128 block scales.
#include "common.h"
#include "kernels.h"

#include <algorithm>

namespace moe {

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
    const float sig = 1.0f / (1.0f + __expf(-g8[i]));
    dg[i] = d8[i] * v8[i] * sig * (1.0f + g8[i] * (1.0f - sig));
    dv[i] = d8[i] * g8[i] * sig;
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
