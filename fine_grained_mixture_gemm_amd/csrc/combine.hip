// Combine (DeepSeek Technical Report: MoE Architecture, 1.1 and 5.3 [1]):
//   h_t = u_t + y_shared_t + sum_k g_{t,k} * y[row_of(t,k)]
// summed in fp32 in that order (k ascending = expert ascending), rounded once to the output dtype.
// A pair that dispatch dropped (row_of = -1: no routed expert, or a repeated one) adds nothing.
// One block per token (d/16 threads rounded up to whole waves, 64 to 1024); each thread reads and writes
// 16-byte pieces of the rows, so every row access is a contiguous, coalesced sweep. A thread issues all
// the loads of a piece (u, the shared row, up to 8 routed rows) before it adds any of them.
//
// Bias update (same report, 3.3): b_i - gamma for an overloaded expert, b_i + gamma for an
// underloaded one, unchanged at the mean load; decided in integers as counts_i * E against T * K.
#include <algorithm>

#include "common.h"
#include "kernels.h"

namespace moe {

constexpr int kCombineMaxK = 8;   // routed rows held in registers at once

// BF16: u and h are bf16 (else fp32); YBF16: the expert outputs are bf16 (else fp32).
template <bool BF16, bool YBF16>
__global__ __launch_bounds__(1024) void combine_rows(const void* __restrict__ u_, const void* __restrict__ yr_,
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
  // 16-byte words per 8 elements of u / h and of the expert outputs
  constexpr int UW = BF16 ? 1 : 2, YW = YBF16 ? 1 : 2;
  auto unpack = [](const uint4 (&w)[2], bool bf, float (&v)[8]) {
    const uint32_t x[8] = {w[0].x, w[0].y, w[0].z, w[0].w, w[1].x, w[1].y, w[1].z, w[1].w};
#pragma unroll
    for (int i = 0; i < 8; ++i)
      v[i] = bf ? __uint_as_float(i & 1 ? x[i / 2] & 0xFFFF0000u : x[i / 2] << 16) : __uint_as_float(x[i]);
  };
  auto words = [](const void* p, size_t byte_off, int n, uint4 (&w)[2]) {
    const uint4* q = reinterpret_cast<const uint4*>(static_cast<const uint8_t*>(p) + byte_off);
    w[0] = q[0];
    if (n > 1) w[1] = q[1];
  };
  for (int c = threadIdx.x; c < nvec; c += blockDim.x) {
    const size_t col = (size_t)c * 8;
    float acc[8], y[8];
    if (K <= kCombineMaxK) {
      // every load of this piece (u, the shared row, the routed rows) is issued before any of them is used,
      // so a piece waits for one memory round trip; the sums keep their order
      uint4 ru[2] = {}, rs[2] = {}, ry[kCombineMaxK][2] = {};
      int rows[kCombineMaxK];
#pragma unroll
      for (int k = 0; k < kCombineMaxK; ++k) rows[k] = k < K ? s_row[k] : -1;
      words(u_, ((size_t)t * d + col) * (BF16 ? 2 : 4), UW, ru);
      if (ys_) words(ys_, ((size_t)t * d + col) * (YBF16 ? 2 : 4), YW, rs);
#pragma unroll
      for (int k = 0; k < kCombineMaxK; ++k)
        if (rows[k] >= 0) words(yr_, ((size_t)rows[k] * d + col) * (YBF16 ? 2 : 4), YW, ry[k]);
      unpack(ru, BF16, acc);
      if (ys_) {
        unpack(rs, YBF16, y);
#pragma unroll
        for (int i = 0; i < 8; ++i) acc[i] += y[i];
      }
#pragma unroll
      for (int k = 0; k < kCombineMaxK; ++k) {
        if (rows[k] < 0) continue;
        const float g = s_g[k];
        unpack(ry[k], YBF16, y);
#pragma unroll
        for (int i = 0; i < 8; ++i) acc[i] = fmaf(g, y[i], acc[i]);
      }
    } else {
      load8(u_, BF16, (size_t)t * d + col, acc);
      if (ys_) {
        load8(ys_, YBF16, (size_t)t * d + col, y);
#pragma unroll
        for (int i = 0; i < 8; ++i) acc[i] += y[i];
      }
      for (int k = 0; k < K; ++k) {
        if (s_row[k] < 0) continue;
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
    for (int k = 0; k < K; ++k)
      if (s_row[k] >= 0) acc = fmaf(s_g[k], load1(yr_, YBF16, (size_t)s_row[k] * d + c), acc);
    if constexpr (BF16) static_cast<uint16_t*>(h_)[(size_t)t * d + c] = f32_to_bf16(acc);
    else static_cast<float*>(h_)[(size_t)t * d + c] = acc;
  }
}

hipError_t launch_combine(const void* u, bool bf16, const void* y_routed, const void* y_shared, bool y_bf16,
                          const int32_t* row_of, const float* topk_w, int T, int d, int K, void* h, hipStream_t s) {
  if (T == 0) return hipSuccess;
  // about two 8-element pieces of the row per thread, so that few threads run a third round
  const int nt = std::min(1024, std::max(64, ((d / 8 + 1) / 2 + 63) / 64 * 64));
  if (bf16 && y_bf16) combine_rows<true, true><<<T, nt, 0, s>>>(u, y_routed, y_shared, row_of, topk_w, d, K, h);
  else if (bf16) combine_rows<true, false><<<T, nt, 0, s>>>(u, y_routed, y_shared, row_of, topk_w, d, K, h);
  else if (!y_bf16) combine_rows<false, false><<<T, nt, 0, s>>>(u, y_routed, y_shared, row_of, topk_w, d, K, h);
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

// Zero `bytes` bytes at p (a small fill kernel instead of a memset node, so that a captured graph replays it
// like any other kernel).
__global__ __launch_bounds__(256) void zero_fill(uint8_t* __restrict__ p, size_t bytes) {
  const size_t n16 = bytes / 16, stride = (size_t)gridDim.x * blockDim.x;
  const size_t t = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  const bool aligned = (reinterpret_cast<uintptr_t>(p) & 15) == 0;
  if (aligned) {
    for (size_t i = t; i < n16; i += stride) reinterpret_cast<uint4*>(p)[i] = make_uint4(0, 0, 0, 0);
    for (size_t i = n16 * 16 + t; i < bytes; i += stride) p[i] = 0;
  } else {
    for (size_t i = t; i < bytes; i += stride) p[i] = 0;
  }
}

hipError_t launch_zero_fill(void* p, size_t bytes, hipStream_t s) {
  if (bytes == 0) return hipSuccess;
  const size_t blocks = std::min<size_t>((bytes / 16 + 255) / 256 + 1, 4096);
  zero_fill<<<(unsigned)blocks, 256, 0, s>>>(static_cast<uint8_t*>(p), bytes);
  return hipGetLastError();
}

hipError_t launch_bias_update(const int32_t* counts, int E, long long TK, float gamma, float* bias, hipStream_t s) {
  bias_update_kernel<<<cdiv(E, 256), 256, 0, s>>>(counts, E, TK, gamma, bias);
  return hipGetLastError();
}

}  // namespace moe
