// Combine (DeepSeek Technical Report: MoE Architecture, 1.1 and 5.3 [1]):
//   h_t = u_t + y_shared_t + sum_k g_{t,k} * y[row_of(t,k)]
// summed in fp32 in that order (k ascending = expert ascending), rounded once to the output dtype.
// One 256-thread block per token; each thread reads and writes 16-byte pieces of the rows, so every
// row access is a contiguous, coalesced sweep.
//
// Bias update (same report, 3.3): b_i - gamma for an overloaded expert, b_i + gamma for an
// underloaded one, unchanged at the mean load; decided in integers as counts_i * E against T * K.
#include "common.h"
#include "kernels.h"

namespace moe {

constexpr int kCombineMaxK = 8;   // routed rows held in registers at once (bf16 expert outputs)

// BF16: u and h are bf16 (else fp32); YBF16: the expert outputs are bf16 (else fp32).
template <bool BF16, bool YBF16>
__global__ __launch_bounds__(256) void combine_rows(const void* __restrict__ u_, const void* __restrict__ yr_,
                                                    const void* __restrict__ ys_, const int32_t* __restrict__ row_of,
                                                    const float* __restrict__ topk_w, int d, int K,
                                                    void* __restrict__ h_) {
  __shared__ int s_row[16];
  __shared__ float s_g[16];
  const int t = blockIdx.x;
  if (threadIdx.x < K) {
    s_row[threadIdx.x] = row_of[(size_t)t * K + threadIdx.x];
    s_g[threadIdx.x] = topk_w[(size_t)t * K + threadIdx.x];
  }
  __syncthreads();
  // 8 consecutive elements per step; vector loads when every row start stays 16-byte aligned
  const bool vec = (d % 8 == 0);
  auto load8 = [&](const void* p, bool bf, size_t off, float (&v)[8]) {
    if (bf) {
      const uint4 r = *reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(p) + off);
      const uint32_t w[4] = {r.x, r.y, r.z, r.w};
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        v[2 * i] = __uint_as_float(w[i] << 16);
        v[2 * i + 1] = __uint_as_float(w[i] & 0xFFFF0000u);
      }
    } else {
      const float4 a = *reinterpret_cast<const float4*>(static_cast<const float*>(p) + off);
      const float4 b = *reinterpret_cast<const float4*>(static_cast<const float*>(p) + off + 4);
      v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w; v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
    }
  };
  auto load1 = [&](const void* p, bool bf, size_t off) -> float {
    return bf ? bf16_to_f32(static_cast<const uint16_t*>(p)[off]) : static_cast<const float*>(p)[off];
  };
  const int nvec = vec ? d / 8 : 0;
  for (int c = threadIdx.x; c < nvec; c += blockDim.x) {
    const size_t col = (size_t)c * 8;
    float acc[8], y[8];
    load8(u_, BF16, (size_t)t * d + col, acc);
    if (ys_) {
      load8(ys_, YBF16, (size_t)t * d + col, y);
#pragma unroll
      for (int i = 0; i < 8; ++i) acc[i] += y[i];
    }
    if (YBF16 && K <= kCombineMaxK) {
      // every routed row's piece is requested before the first is used (K loads in flight), then the
      // rows are added in order
      uint4 raw[kCombineMaxK];
#pragma unroll
      for (int k = 0; k < kCombineMaxK; ++k)
        if (k < K) raw[k] = *reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(yr_) + (size_t)s_row[k] * d + col);
#pragma unroll
      for (int k = 0; k < kCombineMaxK; ++k) {
        if (k >= K) break;
        const float g = s_g[k];
        const uint32_t w[4] = {raw[k].x, raw[k].y, raw[k].z, raw[k].w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          acc[2 * i] = fmaf(g, __uint_as_float(w[i] << 16), acc[2 * i]);
          acc[2 * i + 1] = fmaf(g, __uint_as_float(w[i] & 0xFFFF0000u), acc[2 * i + 1]);
        }
      }
    } else {
      for (int k = 0; k < K; ++k) {
        load8(yr_, YBF16, (size_t)s_row[k] * d + col, y);
        const float g = s_g[k];
#pragma unroll
        for (int i = 0; i < 8; ++i) acc[i] = fmaf(g, y[i], acc[i]);
      }
    }
    if constexpr (BF16) {
      uint4 o;
      o.x = uint32_t(f32_to_bf16(acc[0])) | (uint32_t(f32_to_bf16(acc[1])) << 16);
      o.y = uint32_t(f32_to_bf16(acc[2])) | (uint32_t(f32_to_bf16(acc[3])) << 16);
      o.z = uint32_t(f32_to_bf16(acc[4])) | (uint32_t(f32_to_bf16(acc[5])) << 16);
      o.w = uint32_t(f32_to_bf16(acc[6])) | (uint32_t(f32_to_bf16(acc[7])) << 16);
      *reinterpret_cast<uint4*>(static_cast<uint16_t*>(h_) + (size_t)t * d + col) = o;
    } else {
      float* hp = static_cast<float*>(h_) + (size_t)t * d + col;
      *reinterpret_cast<float4*>(hp) = make_float4(acc[0], acc[1], acc[2], acc[3]);
      *reinterpret_cast<float4*>(hp + 4) = make_float4(acc[4], acc[5], acc[6], acc[7]);
    }
  }
  // columns past the last full group of 8
  for (int c = nvec * 8 + threadIdx.x; c < d; c += blockDim.x) {
    float acc = load1(u_, BF16, (size_t)t * d + c);
    if (ys_) acc += load1(ys_, YBF16, (size_t)t * d + c);
    for (int k = 0; k < K; ++k) acc = fmaf(s_g[k], load1(yr_, YBF16, (size_t)s_row[k] * d + c), acc);
    if constexpr (BF16) static_cast<uint16_t*>(h_)[(size_t)t * d + c] = f32_to_bf16(acc);
    else static_cast<float*>(h_)[(size_t)t * d + c] = acc;
  }
}

hipError_t launch_combine(const void* u, bool bf16, const void* y_routed, const void* y_shared, bool y_bf16,
                          const int32_t* row_of, const float* topk_w, int T, int d, int K, void* h, hipStream_t s) {
  if (T == 0) return hipSuccess;
  if (bf16 && y_bf16) combine_rows<true, true><<<T, 256, 0, s>>>(u, y_routed, y_shared, row_of, topk_w, d, K, h);
  else if (bf16) combine_rows<true, false><<<T, 256, 0, s>>>(u, y_routed, y_shared, row_of, topk_w, d, K, h);
  else if (!y_bf16) combine_rows<false, false><<<T, 256, 0, s>>>(u, y_routed, y_shared, row_of, topk_w, d, K, h);
  else return hipErrorInvalidValue;
  return hipGetLastError();
}

__global__ void bias_update_kernel(const int32_t* __restrict__ counts, int E, long long TK, float gamma,
                                   float* __restrict__ bias) {
  const int e = blockIdx.x * blockDim.x + threadIdx.x;
  if (e >= E) return;
  const long long load = (long long)counts[e] * E;
  const float b = bias[e];
  if (load > TK) bias[e] = b - gamma;
  else if (load < TK) bias[e] = b + gamma;
}

hipError_t launch_bias_update(const int32_t* counts, int E, long long TK, float gamma, float* bias, hipStream_t s) {
  bias_update_kernel<<<cdiv(E, 256), 256, 0, s>>>(counts, E, TK, gamma, bias);
  return hipGetLastError();
}

}  // namespace moe
