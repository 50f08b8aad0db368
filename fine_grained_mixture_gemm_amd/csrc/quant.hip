// Fine-grained E4M3 quantizers (DeepSeek Technical Report: MoE Architecture, 3.6): activations per
// row per 128 columns, weights per 128x128 block. Scale rule: s = amax/448 and inv = 448/amax, both
// correctly rounded fp32 divisions (s = inv = 1 for an all-zero tile), q = E4M3(x * inv) nearest-even
// with saturation.
#include "common.h"
#include "kernels.h"
#include "tiles.h"

namespace moe {

// 8 lanes per 128-column group, 16 consecutive elements (one or more 16-byte loads, one 16-byte store)
// per lane; one 256-thread block covers 32 groups (4096 columns of one row, or several rows when cols is
// smaller).
template <typename TX>
__device__ __forceinline__ void quant_act_group(const TX* __restrict__ x, int rows, int cols, uint8_t* __restrict__ q,
                                                float* __restrict__ scales, long long group) {
  const int groups_per_row = cols / 128;
  if (group >= (long long)rows * groups_per_row) return;   // 8-lane groups exit together
  const int row = (int)(group / groups_per_row), gc = (int)(group % groups_per_row);
  const int sub = threadIdx.x & 7;
  const size_t base = (size_t)row * cols + (size_t)gc * 128 + sub * 16;
  float v[16];
  if constexpr (sizeof(TX) == 2) {
    const uint4 r0 = *reinterpret_cast<const uint4*>(x + base);
    const uint4 r1 = *reinterpret_cast<const uint4*>(x + base + 8);
    const uint32_t w[8] = {r0.x, r0.y, r0.z, r0.w, r1.x, r1.y, r1.z, r1.w};
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      v[2 * i] = __uint_as_float(w[i] << 16);
      v[2 * i + 1] = __uint_as_float(w[i] & 0xFFFF0000u);
    }
  } else {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float4 a = *reinterpret_cast<const float4*>(x + base + 4 * i);
      v[4 * i] = a.x; v[4 * i + 1] = a.y; v[4 * i + 2] = a.z; v[4 * i + 3] = a.w;
    }
  }
  float amax = 0.f;
#pragma unroll
  for (int i = 0; i < 16; ++i) amax = fmaxf(amax, fabsf(v[i]));
#pragma unroll
  for (int o = 4; o > 0; o >>= 1) amax = fmaxf(amax, __shfl_xor(amax, o, 64));
  float s, inv;
  e4m3_scales(amax, s, inv);
  uint4 out;
  out.x = f32x4_to_e4m3x4(v[0] * inv, v[1] * inv, v[2] * inv, v[3] * inv);
  out.y = f32x4_to_e4m3x4(v[4] * inv, v[5] * inv, v[6] * inv, v[7] * inv);
  out.z = f32x4_to_e4m3x4(v[8] * inv, v[9] * inv, v[10] * inv, v[11] * inv);
  out.w = f32x4_to_e4m3x4(v[12] * inv, v[13] * inv, v[14] * inv, v[15] * inv);
  *reinterpret_cast<uint4*>(q + base) = out;
  if (sub == 0) scales[(size_t)row * groups_per_row + gc] = s;
}

template <typename TX>
__global__ __launch_bounds__(256) void quant_act_1x128(const TX* __restrict__ x, int rows, int cols,
                                                       uint8_t* __restrict__ q, float* __restrict__ scales) {
  quant_act_group(x, rows, cols, q, scales, (long long)blockIdx.x * 32 + (threadIdx.x >> 3));
}

// The forward's bf16 activations before the matrix-core GEMMs: block 0 computes the tile schedule of the
// two grouped launches (it needs only the dispatch offsets) while the other blocks quantize, 64 groups of
// 128 elements per 512-thread block; one launch instead of two in a row.
__global__ __launch_bounds__(512) void quant_act_schedule(const uint16_t* __restrict__ x, int rows, int cols,
                                                          uint8_t* __restrict__ q, float* __restrict__ scales,
                                                          SchedArgs sa) {
  if (blockIdx.x == 0) {
    schedule_mfma_block(sa.offsets, sa.E, sa.T, sa.bm, sa.nt_r[0], sa.nt_s[0], sa.nt_r[1], sa.nt_s[1], sa.mt_prefix,
                        sa.xrange, sa.xcount);
    return;
  }
  quant_act_group(x, rows, cols, q, scales, (long long)(blockIdx.x - 1) * 64 + (threadIdx.x >> 3));
}

// One 256-thread block per 128x128 block: each thread handles 64 elements (half a row).
__global__ __launch_bounds__(256) void quant_weight_128x128(const float* __restrict__ w, int rows, int cols,
                                                            uint8_t* __restrict__ q, float* __restrict__ scales) {
  __shared__ float red[4];
  const int cb = blockIdx.x, rb = blockIdx.y, mat = blockIdx.z;
  const int nrb = rows / 128, ncb = cols / 128;
  const size_t mbase = (size_t)mat * rows * cols;
  const int r = rb * 128 + (threadIdx.x >> 1);
  const int c = cb * 128 + (threadIdx.x & 1) * 64;
  const float* src = w + mbase + (size_t)r * cols + c;
  float v[64];
  float amax = 0.f;
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const float4 a = reinterpret_cast<const float4*>(src)[i];
    v[4 * i] = a.x; v[4 * i + 1] = a.y; v[4 * i + 2] = a.z; v[4 * i + 3] = a.w;
    amax = fmaxf(amax, fmaxf(fmaxf(fabsf(a.x), fabsf(a.y)), fmaxf(fabsf(a.z), fabsf(a.w))));
  }
  amax = wave_max(amax);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = amax;
  __syncthreads();
  amax = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
  float s, inv;
  e4m3_scales(amax, s, inv);
  uint8_t* dst = q + mbase + (size_t)r * cols + c;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    uint4 o;
    o.x = f32x4_to_e4m3x4(v[16 * i + 0] * inv, v[16 * i + 1] * inv, v[16 * i + 2] * inv, v[16 * i + 3] * inv);
    o.y = f32x4_to_e4m3x4(v[16 * i + 4] * inv, v[16 * i + 5] * inv, v[16 * i + 6] * inv, v[16 * i + 7] * inv);
    o.z = f32x4_to_e4m3x4(v[16 * i + 8] * inv, v[16 * i + 9] * inv, v[16 * i + 10] * inv, v[16 * i + 11] * inv);
    o.w = f32x4_to_e4m3x4(v[16 * i + 12] * inv, v[16 * i + 13] * inv, v[16 * i + 14] * inv, v[16 * i + 15] * inv);
    reinterpret_cast<uint4*>(dst)[i] = o;
  }
  if (threadIdx.x == 0) scales[(size_t)mat * nrb * ncb + (size_t)rb * ncb + cb] = s;
}

// 64 rows per block: their scales are read row by row (contiguous) into LDS and written block by block.
// One launch does up to two copies: blocks below nb1 the first (gathered through perm), the rest the second.
struct ScaleCopy {
  const int32_t* perm;
  const int32_t* n_rows;
  int rows;
  float* out;
  int ld;
};

__global__ __launch_bounds__(256) void scales_by_block(const float* __restrict__ xs, int kblk, ScaleCopy c1, int nb1,
                                                       ScaleCopy c2) {
  __shared__ float tile[64][65];
  __shared__ int src[64];
  const bool first = (int)blockIdx.x < nb1;
  const ScaleCopy& c = first ? c1 : c2;
  const int r0 = (first ? blockIdx.x : blockIdx.x - nb1) * 64;
  const int n = c.perm ? min(*c.n_rows, c.rows) : c.rows;
  if (r0 >= n) return;
  const int nr = min(64, n - r0);
  if (threadIdx.x < nr) src[threadIdx.x] = c.perm ? c.perm[r0 + threadIdx.x] : r0 + threadIdx.x;
  __syncthreads();
  for (int kb0 = 0; kb0 < kblk; kb0 += 64) {
    const int kc = min(64, kblk - kb0);
    for (int i = threadIdx.x; i < nr * kc; i += 256) {
      const int rr = i / kc, kb = i - rr * kc;
      tile[rr][kb] = xs[(size_t)src[rr] * kblk + kb0 + kb];
    }
    __syncthreads();
    for (int i = threadIdx.x; i < 64 * kc; i += 256) {
      const int kb = i >> 6, rr = i & 63;
      if (rr < nr) c.out[(size_t)(kb0 + kb) * c.ld + r0 + rr] = tile[rr][kb];
    }
    __syncthreads();
  }
}

hipError_t launch_scales_by_block(const float* xs, int kblk, const int32_t* perm, const int32_t* n_rows, int rows,
                                  float* out, int ld, int rows2, float* out2, int ld2, hipStream_t s) {
  if (kblk == 0 || rows + rows2 == 0) return hipSuccess;
  const int nb1 = (rows + 63) / 64, nb2 = (rows2 + 63) / 64;
  scales_by_block<<<nb1 + nb2, 256, 0, s>>>(xs, kblk, ScaleCopy{perm, n_rows, rows, out, ld}, nb1,
                                            ScaleCopy{nullptr, nullptr, rows2, out2, ld2});
  return hipGetLastError();
}

hipError_t launch_quant_act(const void* x, bool x_bf16, int rows, int cols, uint8_t* q, float* scales, hipStream_t s) {
  if (rows == 0) return hipSuccess;
  const long long groups = (long long)rows * (cols / 128);
  const unsigned nb = (unsigned)((groups + 31) / 32);
  if (x_bf16) quant_act_1x128<uint16_t><<<nb, 256, 0, s>>>((const uint16_t*)x, rows, cols, q, scales);
  else quant_act_1x128<float><<<nb, 256, 0, s>>>((const float*)x, rows, cols, q, scales);
  return hipGetLastError();
}

hipError_t launch_quant_act_schedule(const void* x, int rows, int cols, uint8_t* q, float* scales, const SchedArgs& sa,
                                     hipStream_t s) {
  const long long groups = (long long)rows * (cols / 128);
  const unsigned nb = 1 + (unsigned)((groups + 63) / 64);
  quant_act_schedule<<<nb, 512, 0, s>>>((const uint16_t*)x, rows, cols, q, scales, sa);
  return hipGetLastError();
}

hipError_t launch_quant_weight(const float* w, int batch, int rows, int cols, uint8_t* q, float* scales, hipStream_t s) {
  if (batch == 0) return hipSuccess;
  dim3 grid(cols / 128, rows / 128, batch);
  quant_weight_128x128<<<grid, 256, 0, s>>>(w, rows, cols, q, scales);
  return hipGetLastError();
}

}  // namespace moe
