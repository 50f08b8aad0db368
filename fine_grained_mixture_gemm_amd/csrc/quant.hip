// Fine-grained E4M3 quantizers (DeepSeek Technical Report: MoE Architecture, 3.6): activations per
// row per 128 columns, weights per 128x128 block. Scale rule: s = amax/448 and inv = 448/amax, both
// correctly rounded fp32 divisions (s = inv = 1 for an all-zero tile), q = E4M3(x * inv) nearest-even
// with saturation.
#include "common.h"
#include "kernels.h"

namespace moe {

// 16 lanes per 128-column group, 8 consecutive elements per lane; one 256-thread block covers
// 16 groups (2048 columns of one row, or several rows when cols is smaller).
template <typename TX>
__global__ __launch_bounds__(256) void quant_act_1x128(const TX* __restrict__ x, int rows, int cols,
                                                       uint8_t* __restrict__ q, float* __restrict__ scales) {
  const int groups_per_row = cols / 128;
  const long long group = (long long)blockIdx.x * 16 + (threadIdx.x >> 4);
  if (group >= (long long)rows * groups_per_row) return;   // 16-lane groups exit together
  const int row = (int)(group / groups_per_row), gc = (int)(group % groups_per_row);
  const int sub = threadIdx.x & 15;
  const size_t base = (size_t)row * cols + (size_t)gc * 128 + sub * 8;
  float v[8];
  if constexpr (sizeof(TX) == 2) {
    const uint4 raw = *reinterpret_cast<const uint4*>(x + base);
    const uint32_t w[4] = {raw.x, raw.y, raw.z, raw.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      v[2 * i] = __uint_as_float(w[i] << 16);
      v[2 * i + 1] = __uint_as_float(w[i] & 0xFFFF0000u);
    }
  } else {
    const float4 a = *reinterpret_cast<const float4*>(x + base);
    const float4 b = *reinterpret_cast<const float4*>(x + base + 4);
    v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w; v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
  }
  float amax = 0.f;
#pragma unroll
  for (int i = 0; i < 8; ++i) amax = fmaxf(amax, fabsf(v[i]));
#pragma unroll
  for (int o = 8; o > 0; o >>= 1) amax = fmaxf(amax, __shfl_xor(amax, o, 64));
  float s, inv;
  e4m3_scales(amax, s, inv);
  uint2 out;
  out.x = f32x4_to_e4m3x4(v[0] * inv, v[1] * inv, v[2] * inv, v[3] * inv);
  out.y = f32x4_to_e4m3x4(v[4] * inv, v[5] * inv, v[6] * inv, v[7] * inv);
  *reinterpret_cast<uint2*>(q + base) = out;
  if (sub == 0) scales[(size_t)row * groups_per_row + gc] = s;
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

hipError_t launch_quant_act(const void* x, bool x_bf16, int rows, int cols, uint8_t* q, float* scales, hipStream_t s) {
  if (rows == 0) return hipSuccess;
  const long long groups = (long long)rows * (cols / 128);
  const unsigned nb = (unsigned)((groups + 15) / 16);
  if (x_bf16) quant_act_1x128<uint16_t><<<nb, 256, 0, s>>>((const uint16_t*)x, rows, cols, q, scales);
  else quant_act_1x128<float><<<nb, 256, 0, s>>>((const float*)x, rows, cols, q, scales);
  return hipGetLastError();
}

hipError_t launch_quant_weight(const float* w, int batch, int rows, int cols, uint8_t* q, float* scales, hipStream_t s) {
  if (batch == 0) return hipSuccess;
  dim3 grid(cols / 128, rows / 128, batch);
  quant_weight_128x128<<<grid, 256, 0, s>>>(w, rows, cols, q, scales);
  return hipGetLastError();
}

}  // namespace moe
