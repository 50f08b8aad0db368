// Router: gate logits, scores, top-K selection and gates.
//
// DeepSeek Technical Report: MoE Architecture, 2.3 (g = Softmax_i(u_t^T e_i), then Top-K) and 3.3
// (s = Sigmoid(u_t^T e_i); expert i is selected when s_i + b_i is among the K largest keys, and its gate
// is the raw s_i). Keys are compared in fp32; a token whose K-th and (K+1)-th keys are closer than
// `delta` is selected again from fp64 logits, so the selected set is the exact top-K of the keys.
#include <type_traits>

#include "common.h"
#include "kernels.h"

namespace moe {

// ------------------------------------------------------------------ logits on the vector ALUs
// z[t, e] = sum_k u[t, k] * wg[e, k] + off[e]; 64 tokens x 64 experts per block, 4 x 4 per thread.
// The products of fp32 / bf16 inputs are exact in fp64 and accumulate in fp64 (same vector rate as
// unpacked fp32); z is rounded to fp32 once. With few tokens (a decode step) blockIdx.z takes one slice
// [z klen, (z + 1) klen) of d and stores its fp64 partial sum, and router_logits_sum adds the slices in
// order, so the result does not depend on how the blocks are scheduled. Blocks of the first 64 experts
// also add up the squares of their token rows over their slice (un2part[slice][t], for the recheck
// margin; nullptr: not wanted).
template <typename TU>
__global__ __launch_bounds__(256) void router_logits_valu(const TU* __restrict__ u, const float* __restrict__ wg,
                                                          const float* __restrict__ off, int T, int E, int d,
                                                          int klen, float* __restrict__ z, double* __restrict__ zpart,
                                                          int* __restrict__ recheck_count, float* __restrict__ un2part) {
  __shared__ float As[32][68];
  __shared__ float Bs[32][68];
  const int tid = threadIdx.x;
  const int t0 = blockIdx.x * 64, e0 = blockIdx.y * 64;
  if (blockIdx.x == 0 && blockIdx.y == 0 && blockIdx.z == 0 && tid == 0) *recheck_count = 0;
  const int tx = tid & 15, ty = tid >> 4;
  double acc[4][4] = {};
  const int lr = tid >> 2, lk = (tid & 3) * 8;
  const int kb = blockIdx.z * klen, ke = min(d, kb + klen);
  const bool norms = un2part != nullptr && blockIdx.y == 0;
  float sa = 0.f;                         // squares of this thread's pieces of token row t0 + lr
  for (int k0 = kb; k0 < ke; k0 += 32) {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int k = k0 + lk + i;
      float a = 0.f, b = 0.f;
      if (t0 + lr < T && k < ke) {
        if constexpr (sizeof(TU) == 2) a = bf16_to_f32(u[(size_t)(t0 + lr) * d + k]);
        else a = u[(size_t)(t0 + lr) * d + k];
      }
      if (e0 + lr < E && k < ke) b = wg[(size_t)(e0 + lr) * d + k];
      As[lk + i][lr] = a;
      Bs[lk + i][lr] = b;
      if (norms) sa = fmaf(a, a, sa);
    }
    __syncthreads();
#pragma unroll 8
    for (int k = 0; k < 32; ++k) {
      float a[4], b[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) a[i] = As[k][ty * 4 + i];
#pragma unroll
      for (int j = 0; j < 4; ++j) b[j] = Bs[k][tx * 4 + j];
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = fma((double)a[i], (double)b[j], acc[i][j]);
    }
    __syncthreads();
  }
  if (norms) {
    // the 4 threads 4 lr .. 4 lr + 3 hold the pieces of row lr
    sa += __shfl_xor(sa, 1, 64);
    sa += __shfl_xor(sa, 2, 64);
    if ((tid & 3) == 0 && t0 + lr < T) un2part[(size_t)blockIdx.z * T + t0 + lr] = sa;
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int t = t0 + ty * 4 + i;
    if (t >= T) continue;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int e = e0 + tx * 4 + j;
      if (e >= E) continue;
      if (zpart) zpart[((size_t)blockIdx.z * T + t) * E + e] = acc[i][j];
      else z[(size_t)t * E + e] = (float)(acc[i][j] + (off ? (double)off[e] : 0.0));
    }
  }
}

// z[t, e] = fp32(sum over slices s = 0.. of zpart[s, t, e] + off[e]), the slices added in order.
__global__ __launch_bounds__(256) void router_logits_sum(const double* __restrict__ zpart, int ksplit, int T, int E,
                                                         const float* __restrict__ off, float* __restrict__ z) {
  const size_t n = (size_t)T * E;
  for (size_t i = (size_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (size_t)gridDim.x * 256) {
    double acc = 0.0;
#pragma unroll 8
    for (int s = 0; s < ksplit; ++s) acc += zpart[(size_t)s * n + i];
    z[i] = (float)(acc + (off ? (double)off[i % E] : 0.0));
  }
}

// ------------------------------------------------------------------ fp32-accurate logits on MFMA
// w_gate is split exactly into three bf16 parts, w = hi + mid + lo (hi and mid truncate, lo holds the
// last 8 significant bits); bf16 x bf16 products are exact in fp32, so the three bf16 GEMMs
// accumulated in fp32 give the fp32 product of the bf16 tokens with the fp32 centroids.
__device__ __forceinline__ void split_bf16x3(float w, uint16_t& hi, uint16_t& mid, uint16_t& lo) {
  const uint32_t hb = __float_as_uint(w) & 0xFFFF0000u;
  const float r1 = w - __uint_as_float(hb);
  const uint32_t mb = __float_as_uint(r1) & 0xFFFF0000u;
  const float r2 = r1 - __uint_as_float(mb);
  hi = (uint16_t)(hb >> 16);
  mid = (uint16_t)(mb >> 16);
  lo = f32_to_bf16(r2);
}

// One block per routed expert: wn2[e] = |e_e|^2 (for the recheck margin) and, with SPLIT, the three bf16
// parts of the centroid row for the MFMA logits (parts [3][E][d]).
template <bool SPLIT>
__global__ __launch_bounds__(256) void router_prep_wg(const float* __restrict__ wg, int E, int d,
                                                      float* __restrict__ wn2, uint16_t* __restrict__ parts) {
  __shared__ float part[4];
  const int e = blockIdx.x;
  const size_t n = (size_t)E * d;
  float s = 0.f;
  if (d % 4 == 0) {
    // 16-byte pieces: thread tid takes pieces p = tid, tid + 256, ... (elements 4p..4p+3), eight pieces
    // in flight at once; its squares are added in element order
    constexpr int kG = 8;
    const int np = d / 4;
    const float4* w4 = reinterpret_cast<const float4*>(wg + (size_t)e * d);
    for (int p0 = threadIdx.x; p0 < np; p0 += 256 * kG) {
      float4 v[kG];
#pragma unroll
      for (int q = 0; q < kG; ++q) {
        const int p = p0 + 256 * q;
        v[q] = p < np ? w4[p] : make_float4(0.f, 0.f, 0.f, 0.f);
      }
#pragma unroll
      for (int q = 0; q < kG; ++q) {
        const int p = p0 + 256 * q;
        if (p < np) {
          const float x[4] = {v[q].x, v[q].y, v[q].z, v[q].w};
#pragma unroll
          for (int r = 0; r < 4; ++r) s = fmaf(x[r], x[r], s);
          if constexpr (SPLIT) {
            ushort4 h, m, l;
            split_bf16x3(x[0], h.x, m.x, l.x);
            split_bf16x3(x[1], h.y, m.y, l.y);
            split_bf16x3(x[2], h.z, m.z, l.z);
            split_bf16x3(x[3], h.w, m.w, l.w);
            const size_t i = (size_t)e * d + 4 * (size_t)p;
            *reinterpret_cast<ushort4*>(parts + i) = h;
            *reinterpret_cast<ushort4*>(parts + n + i) = m;
            *reinterpret_cast<ushort4*>(parts + 2 * n + i) = l;
          }
        }
      }
    }
  } else {
    // each thread's elements k = tid, tid + 256, ... in groups of 16, all loads of a group in flight at
    // once; the squares are added in k order
    constexpr int kG = 16;
    for (int k0 = threadIdx.x; k0 < d; k0 += 256 * kG) {
      float v[kG];
#pragma unroll
      for (int q = 0; q < kG; ++q) {
        const int k = k0 + 256 * q;
        v[q] = k < d ? wg[(size_t)e * d + k] : 0.f;
      }
#pragma unroll
      for (int q = 0; q < kG; ++q) {
        const int k = k0 + 256 * q;
        if (k < d) {
          const size_t i = (size_t)e * d + k;
          s = fmaf(v[q], v[q], s);
          if constexpr (SPLIT) split_bf16x3(v[q], parts[i], parts[n + i], parts[2 * n + i]);
        }
      }
    }
  }
  s = wave_sum(s);
  if ((threadIdx.x & 63) == 0) part[threadIdx.x >> 6] = s;
  __syncthreads();
  if (threadIdx.x == 0) wn2[e] = (part[0] + part[1]) + (part[2] + part[3]);
}

// 16 TJ tokens x 16 NW experts per block (NW waves); wave w owns experts 16w..16w+15 against all the
// block's tokens. Tokens are staged 64 elements (128 bytes) at a time in a double-buffered XOR-swizzled LDS
// tile; the centroid parts stream from global memory into registers. blockIdx.z takes the slice
// [z klen, (z + 1) klen) of d: with one slice the kernel writes z = sum + off, with several it writes
// the slice's fp32 partial sum to zpart[z] and router_logits_sum32 adds the slices in order.
// Blocks of the first expert tile also add up the squares of their token rows over their slice of d
// (un2part[slice][t], for the recheck margin; nullptr: not wanted).
// Two shapes: 128 tokens x 64 experts (4 waves), and for large batches 256 tokens x 128 experts (8 waves),
// which reads half the tokens and centroid parts from L2 per product.
template <int TJ, int NW, int PF>
__global__ __launch_bounds__(64 * NW) void router_logits_mfma(const uint16_t* __restrict__ u, const uint16_t* __restrict__ parts,
                                                             const float* __restrict__ off, int T, int E, int d,
                                                             int klen, float* __restrict__ z, float* __restrict__ zpart,
                                                             int* __restrict__ recheck_count, float* __restrict__ un2part) {
  constexpr int kTM = 16 * TJ, kThr = 64 * NW;
  constexpr int kQ = kTM * 8 / kThr;   // 16-byte token pieces per thread per stage
  static_assert(kQ * kThr == kTM * 8 && TJ % 8 == 0, "token staging");
  __shared__ __attribute__((aligned(16))) uint8_t lds[2][kTM * 128];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int t0 = blockIdx.x * kTM, e0 = blockIdx.y * (16 * NW);
  if (blockIdx.x == 0 && blockIdx.y == 0 && blockIdx.z == 0 && tid == 0) *recheck_count = 0;
  const size_t n = (size_t)E * d;
  const int s0 = blockIdx.z * (klen / 64), nst = min(d, (int)(blockIdx.z + 1) * klen) / 64 - s0;
  const int erow = min(e0 + 16 * wave + (lane & 15), E - 1);
  const uint8_t* wp = reinterpret_cast<const uint8_t*>(parts + (size_t)erow * d) + 16 * (lane >> 4) + 128 * s0;
  const uint8_t* ub = reinterpret_cast<const uint8_t*>(u);
  uint32_t boff[kQ];
#pragma unroll
  for (int q = 0; q < kQ; ++q) {
    const int id16 = q * kThr + tid;
    const int tok = min(t0 + (id16 >> 3), T - 1);
    boff[q] = (uint32_t)tok * (uint32_t)d * 2u + (id16 & 7) * 16 + 128u * s0;
  }
  f32x4 acc[TJ];
#pragma unroll
  for (int j = 0; j < TJ; ++j) acc[j] = f32x4{0.f, 0.f, 0.f, 0.f};
  // Tokens and centroid parts are loaded PF stages ahead (1 or 2) into two register sets used by even and
  // odd stages (the loop below takes stages in pairs, so each set stays in fixed registers).
  auto load_tokens = [&](int kb, i32x4 (&B)[kQ]) {
#pragma unroll
    for (int q = 0; q < kQ; ++q) B[q] = *reinterpret_cast<const i32x4*>(ub + (size_t)kb * 128 + boff[q]);
  };
  auto load_parts = [&](int kb, i32x4 (&A)[3][2]) {
#pragma unroll
    for (int p = 0; p < 3; ++p) {
      const uint8_t* pp = wp + p * n * 2 + (size_t)kb * 128;
      A[p][0] = *reinterpret_cast<const i32x4*>(pp);
      A[p][1] = *reinterpret_cast<const i32x4*>(pp + 64);
    }
  };
  const int tr = lane & 15, g = lane >> 4;
  const bool norms = un2part != nullptr && blockIdx.y == 0;
  float su[kQ];   // squares of this thread's 8-element pieces of rows (q kThr + tid) / 8
#pragma unroll
  for (int q = 0; q < kQ; ++q) su[q] = 0.f;
  i32x4 B0[kQ], B1[kQ], A0[3][2], A1[3][2];
  load_tokens(0, B0);
  load_parts(0, A0);
  if (PF == 2 && nst > 1) {
    load_tokens(1, B1);
    load_parts(1, A1);
  }
  // B, A: this stage's sets; Bn, An: the next stage's
  auto stage = [&](int kb, i32x4 (&B)[kQ], i32x4 (&A)[3][2], i32x4 (&Bn)[kQ], i32x4 (&An)[3][2]) {
    uint8_t* buf = lds[kb & 1];
#pragma unroll
    for (int q = 0; q < kQ; ++q) {
      const int id16 = q * kThr + tid, row = id16 >> 3, c = id16 & 7;
      *reinterpret_cast<i32x4*>(buf + row * 128 + ((c ^ (row & 7)) * 16)) = B[q];
      if (norms) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float lo = __uint_as_float((uint32_t)B[q][i] << 16), hi = __uint_as_float((uint32_t)B[q][i] & 0xFFFF0000u);
          su[q] = fmaf(hi, hi, fmaf(lo, lo, su[q]));
        }
      }
    }
    __syncthreads();
    if (PF == 2 && kb + 2 < nst) load_tokens(kb + 2, B);
    if (PF == 1 && kb + 1 < nst) {
      load_tokens(kb + 1, Bn);
      load_parts(kb + 1, An);
    }
    // groups of eight token tiles; within a group the tiles are innermost, so consecutive MFMAs update
    // different accumulators
#pragma unroll
    for (int j0 = 0; j0 < TJ; j0 += 8) {
      i32x4 b[8][2];
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const int row = 16 * (j0 + j) + tr;
        b[j][0] = *reinterpret_cast<const i32x4*>(buf + row * 128 + ((g ^ (row & 7)) * 16));
        b[j][1] = *reinterpret_cast<const i32x4*>(buf + row * 128 + (((4 + g) ^ (row & 7)) * 16));
      }
#pragma unroll
      for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int p = 0; p < 3; ++p)
#pragma unroll
          for (int j = 0; j < 8; ++j)
            acc[j0 + j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, A[p][h]),
                                                                  __builtin_bit_cast(bf16x8, b[j][h]), acc[j0 + j], 0, 0, 0);
    }
    if (PF == 2 && kb + 2 < nst) load_parts(kb + 2, A);
  };
  for (int kb = 0; kb < nst; kb += 2) {
    stage(kb, B0, A0, B1, A1);
    if (kb + 1 < nst) stage(kb + 1, B1, A1, B0, A0);
  }
  if (norms) {
    // the 8 threads tid & ~7 .. tid | 7 hold the pieces of one row
#pragma unroll
    for (int q = 0; q < kQ; ++q) {
      float v = su[q];
      v += __shfl_xor(v, 1, 64);
      v += __shfl_xor(v, 2, 64);
      v += __shfl_xor(v, 4, 64);
      const int t = t0 + (q * kThr + tid) / 8;
      if ((tid & 7) == 0 && t < T) un2part[(size_t)blockIdx.z * T + t] = v;
    }
  }
  // lane holds experts 16 wave + 4 (lane >> 4) + r for token 16 j + (lane & 15)
#pragma unroll
  for (int j = 0; j < TJ; ++j) {
    const int t = t0 + 16 * j + (lane & 15);
    if (t >= T) continue;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int e = e0 + 16 * wave + 4 * (lane >> 4) + r;
      if (e >= E) continue;
      if (zpart) zpart[((size_t)blockIdx.z * T + t) * E + e] = acc[j][r];
      else z[(size_t)t * E + e] = acc[j][r] + (off ? off[e] : 0.f);
    }
  }
}

// z[t, e] = fp32(sum over slices s = 0.. of zpart[s, t, e], in order) + off[e].
__global__ __launch_bounds__(256) void router_logits_sum32(const float* __restrict__ zpart, int ks, int T, int E,
                                                           const float* __restrict__ off, float* __restrict__ z) {
  const size_t n = (size_t)T * E;
  for (size_t i = (size_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (size_t)gridDim.x * 256) {
    float acc = zpart[i];
    for (int k = 1; k < ks; ++k) acc += zpart[(size_t)k * n + i];
    z[i] = acc + (off ? off[i % E] : 0.f);
  }
}

void launch_router_logits_mfma(const RouteArgs& a, hipStream_t s) {
  router_prep_wg<true><<<a.E, 256, 0, s>>>(a.wg, a.E, a.d, a.wn2, a.wg_split);
  // several slices of d when one gives fewer than two blocks per CU; their fp32 partial sums live in the
  // space of the fp64 recheck logits (sized for four slices), which are written only later
  const int ks = router_mfma_slices(a.T, a.E, a.d);
  const int klen = cdiv(a.d / 64, ks) * 64;
  float* zp = ks > 1 ? reinterpret_cast<float*>(a.z64) : nullptr;
  if (router_mfma_large(a.T, a.E)) {
    dim3 grid(cdiv(a.T, 256), cdiv(a.E, 128), ks);
    router_logits_mfma<16, 8, 2><<<grid, 512, 0, s>>>((const uint16_t*)a.u, a.wg_split, a.off, a.T, a.E, a.d, klen, a.z,
                                                   zp, a.recheck_count, a.un2);
  } else {
    dim3 grid(cdiv(a.T, 128), cdiv(a.E, 64), ks);
    router_logits_mfma<8, 4, 1><<<grid, 256, 0, s>>>((const uint16_t*)a.u, a.wg_split, a.off, a.T, a.E, a.d, klen, a.z,
                                                  zp, a.recheck_count, a.un2);
  }
  if (ks > 1) {
    const long long nz = (long long)a.T * a.E;
    const long long nb = (nz + 255) / 256;
    router_logits_sum32<<<(unsigned)(nb < 2048 ? nb : 2048), 256, 0, s>>>(zp, ks, a.T, a.E, a.off, a.z);
  }
}

// ------------------------------------------------------------------ recheck margin per token
// The fp32 logits round every partial sum of u_t . e_i; each rounding is proportional to the running sum,
// which is at most |u_t| |e_i| (Cauchy-Schwarz). The base margin holds for |u_t| |e_i| up to sqrt(d) (token
// rows of RMS 1 against centroids of norm 1); a token whose |u_t| max_i |e_i| is larger gets the margin
// scaled by the ratio. wn2[i] = |e_i|^2 comes from router_prep_wg.
// delta * max(1, |u_t| max_i |e_i| / sqrt(d)) for token t, on one wave: |u_t|^2 is the sum of the nsl
// slice partials un2[s][t] the logits kernels wrote (lane l takes slices l, l + 64, ..., then a fixed
// reduction tree).
__device__ __forceinline__ float token_margin(const float* __restrict__ un2, int nsl, int t, int T, int d,
                                              const float* __restrict__ wn2, int E, float delta, int lane) {
  float su = 0.f;
  for (int sl = lane; sl < nsl; sl += 64) su += un2[(size_t)sl * T + t];
  su = wave_sum(su);
  float wm = 0.f;
  for (int e = lane; e < E; e += 64) wm = fmaxf(wm, wn2[e]);
  wm = wave_max(wm);
  return delta * fmaxf(1.f, sqrtf(su * wm / (float)d));
}

// ------------------------------------------------------------------ top-K of one token per wave
__device__ __forceinline__ float f32_unorder(uint32_t o) {
  return __uint_as_float((o & 0x80000000u) ? (o & 0x7FFFFFFFu) : ~o);
}

// Lane r < K ends with the r-th selected expert in `my_e`; returns the gap between the K-th and the
// (K+1)-th largest key (+inf when K == E). Ties go to the lower expert index: the packed value puts the
// complemented index in the low word.
__device__ __forceinline__ float wave_topk_f32(const float key[4], const bool valid[4], int E, int K, int lane,
                                               int& my_e) {
  uint64_t packed[4];
#pragma unroll
  for (int j = 0; j < 4; ++j)
    packed[j] = valid[j] ? ((uint64_t)f32_order(key[j]) << 32) | (uint64_t)(0xFFFFFFFFu - (uint32_t)(lane + 64 * j)) : 0;
  float kth = 0.f, k1 = __builtin_inff();
  const int rounds = K < E ? K + 1 : K;
  my_e = -1;
  for (int r = 0; r < rounds; ++r) {
    uint64_t best = 0;
#pragma unroll
    for (int j = 0; j < 4; ++j) best = packed[j] > best ? packed[j] : best;
    best = wave_max_u64(best);
    const int e = (int)(0xFFFFFFFFu - (uint32_t)best);
    const float kv = f32_unorder((uint32_t)(best >> 32));
    if ((e & 63) == lane) {
#pragma unroll
      for (int j = 0; j < 4; ++j)
        if (j == (e >> 6)) packed[j] = 0;
    }
    if (r < K && lane == r) my_e = e;
    if (r == K - 1) kth = kv;
    if (r == K) k1 = kv;
  }
  // no (K+1)-th key when K == E: the selection is decided by construction
  return rounds > K ? kth - k1 : __builtin_inff();
}

// Group-limited routing on one wave (DeepSeek Technical Report: MoE Architecture, 2.3 device-limited
// routing; 3.2 / 3.8 node-limited routing). Lanes hold the keys of experts lane + 64 j (valid[j]: the
// expert exists). The E experts form G equal contiguous groups; a group scores the largest key of its
// experts; the M best groups are kept (ties to the lower group index) and valid[] is cleared for the
// experts of every other group. Returns the M-th best group score minus the (M+1)-th (+inf when
// M == G): the margin by which the group choice is decided.
template <typename V>
__device__ __forceinline__ V group_limit_wave(const V key[4], bool valid[4], int E, int G, int M, int lane) {
  const V ninf = -__builtin_inf();
  const int gsz = E / G;
  V gsc = ninf;                          // lane g < G: score of group g
  for (int g = 0; g < G; ++g) {
    V m = ninf;
#pragma unroll
    for (int j = 0; j < 4; ++j)
      if (valid[j] && (lane + 64 * j) / gsz == g) m = key[j] > m ? key[j] : m;
    for (int o = 32; o > 0; o >>= 1) {
      const V om = __shfl_xor(m, o, 64);
      m = om > m ? om : m;
    }
    if (lane == g) gsc = m;
  }
  bool cand = lane < G;
  unsigned keep = 0;
  V mth = 0, m1 = ninf;
  const int rounds = M < G ? M + 1 : M;
  for (int r = 0; r < rounds; ++r) {
    V bv = cand ? gsc : ninf;
    int bg = cand ? lane : 0x7FFFFFFF;
    for (int o = 32; o > 0; o >>= 1) {
      const V ov = __shfl_xor(bv, o, 64);
      const int og = __shfl_xor(bg, o, 64);
      if (ov > bv || (ov == bv && og < bg)) {
        bv = ov;
        bg = og;
      }
    }
    if (r < M) {
      keep |= 1u << bg;
      if (lane == bg) cand = false;
      mth = bv;
    } else {
      m1 = bv;
    }
  }
#pragma unroll
  for (int j = 0; j < 4; ++j)
    if (valid[j] && !((keep >> ((lane + 64 * j) / gsz)) & 1u)) valid[j] = false;
  return mth - m1;
}

template <int GATE>
__global__ __launch_bounds__(256) void router_topk(const float* __restrict__ z, int T, int E, int K,
                                                   const float* __restrict__ bias, int renorm, int G, int M,
                                                   float delta, int d,
                                                   const float* __restrict__ un2, int nsl, const float* __restrict__ wn2,
                                                   int32_t* __restrict__ topk_idx, float* __restrict__ topk_w,
                                                   int* __restrict__ recheck_count, int* __restrict__ recheck_list) {
  const int lane = threadIdx.x & 63;
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= T) return;
  float zz[4], key[4], score[4];
  bool valid[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int e = lane + 64 * j;
    valid[j] = e < E;
    zz[j] = valid[j] ? z[(size_t)t * E + e] : -__builtin_inff();
  }
  if (GATE == MOE_GATE_SOFTMAX) {
    float m = -__builtin_inff();
#pragma unroll
    for (int j = 0; j < 4; ++j) m = fmaxf(m, zz[j]);
    m = wave_max(m);
    float p[4], s = 0.f;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      p[j] = valid[j] ? expf(zz[j] - m) : 0.f;
      s += p[j];
    }
    s = wave_sum(s);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      score[j] = p[j] / s;
      key[j] = zz[j];
    }
  } else {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int e = lane + 64 * j;
      score[j] = valid[j] ? 1.0f / (1.0f + expf(-zz[j])) : 0.f;
      key[j] = score[j] + ((bias && valid[j]) ? bias[e] : 0.f);
    }
  }
  // gates above come from every expert; the group limit only narrows the selection
  float ggap = __builtin_inff();
  int n_allowed = E;
  if (G > 0) {
    ggap = group_limit_wave<float>(key, valid, E, G, M, lane);
    n_allowed = M * (E / G);
  }
  int my_e;
  const float gap = fminf(wave_topk_f32(key, valid, n_allowed, K, lane, my_e), ggap);
  // gate of this lane's expert: fetch score[my_e >> 6] from lane my_e & 63
  const int src = my_e < 0 ? 0 : (my_e & 63);
  float g = 0.f;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const float v = __shfl(score[j], src, 64);
    if (my_e >= 0 && j == (my_e >> 6)) g = v;
  }
  if (renorm) g = g / wave_sum(lane < K ? g : 0.f);
  // rank of this lane's expert among the K selected -> ascending order
  int rank = 0;
  for (int q = 0; q < K; ++q) {
    const int eq = __shfl(my_e, q, 64);
    rank += (eq < my_e) ? 1 : 0;
  }
  if (lane < K) {
    topk_idx[(size_t)t * K + rank] = my_e;
    topk_w[(size_t)t * K + rank] = g;
  }
  const float margin = token_margin(un2, nsl, t, T, d, wn2, E, delta, lane);
  if (lane == 0 && gap < margin) {
    const int pos = atomicAdd(recheck_count, 1);
    recheck_list[pos] = t;
  }
}

// ------------------------------------------------------------------ fp64 recheck of close tokens
// Pass 1: fp64 logits of the flagged tokens. Eight blocks per routed expert e hold centroid row e in
// registers (each thread every 256th element, as fp64); block y takes batches y, y + 8, ... of 8 flagged
// tokens (so a handful of flagged tokens does not run as one long chain of batches per expert), reading
// their u elements straight from memory (every element is used once per block, so there is nothing to
// stage; the flagged rows stay in L2 for the other blocks); each of the 8 dot products is reduced in
// fp64. Products of the stored inputs are exact in fp64.
constexpr int kRecheckThreads = 256;
constexpr int kRecheckMaxD = 8192;
constexpr int kRecheckPer = kRecheckMaxD / kRecheckThreads;   // centroid elements per thread (32)
constexpr int kRecheckBatch = 8;                               // flagged tokens per pass
constexpr int kRecheckSplit = 8;                               // blocks per expert, each every 8th batch

template <typename TU>
__global__ __launch_bounds__(kRecheckThreads) void router_recheck_logits(const TU* __restrict__ u,
                                                                         const float* __restrict__ wg,
                                                                         const float* __restrict__ off, int E, int d,
                                                                         const int* __restrict__ recheck_count,
                                                                         const int* __restrict__ recheck_list,
                                                                         double* __restrict__ z64) {
  __shared__ double part[kRecheckBatch][kRecheckThreads / 64];
  const int n = *recheck_count;
  // blockIdx.y takes batches y, y + gridDim.y, ... of the flagged tokens
  if (n <= (int)blockIdx.y * kRecheckBatch) return;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  for (int e = blockIdx.x; e < E; e += gridDim.x) {
    // indices past d are clamped (no branches, so every load can be in flight at once); their centroid
    // values are zero and add nothing
    double w[kRecheckPer];
#pragma unroll
    for (int i = 0; i < kRecheckPer; ++i) {
      const int k = tid + kRecheckThreads * i;
      const double v = (double)wg[(size_t)e * d + min(k, d - 1)];
      w[i] = k < d ? v : 0.0;
    }
    const double o = off ? (double)off[e] : 0.0;
    for (int q0 = blockIdx.y * kRecheckBatch; q0 < n; q0 += gridDim.y * kRecheckBatch) {
      const int nb = min(kRecheckBatch, n - q0);
      double acc[kRecheckBatch];
#pragma unroll
      for (int b = 0; b < kRecheckBatch; ++b) {
        acc[b] = 0.0;
        if (b < nb) {
          const TU* ur = u + (size_t)recheck_list[q0 + b] * d;
          float x[kRecheckPer];
#pragma unroll
          for (int i = 0; i < kRecheckPer; ++i) {
            const int k = min(tid + kRecheckThreads * i, d - 1);
            if constexpr (sizeof(TU) == 2) x[i] = bf16_to_f32(ur[k]);
            else x[i] = ur[k];
          }
#pragma unroll
          for (int i = 0; i < kRecheckPer; ++i) acc[b] = fma((double)x[i], w[i], acc[b]);
        }
      }
#pragma unroll
      for (int b = 0; b < kRecheckBatch; ++b) {
        const double sum = wave_sum(acc[b]);
        if (lane == 0) part[b][wave] = sum;
      }
      __syncthreads();
      if (tid < nb) z64[(size_t)(q0 + tid) * E + e] = ((part[tid][0] + part[tid][1]) + (part[tid][2] + part[tid][3])) + o;
      __syncthreads();                                  // part is written again by the next batch
    }
  }
}

// Pass 2: one wave per flagged token selects again from the fp64 logits and rewrites its outputs.
template <int GATE>
__global__ __launch_bounds__(256) void router_recheck_select(const double* __restrict__ z64, int E, int K,
                                                             const float* __restrict__ bias, int renorm, int G, int M,
                                                             const int* __restrict__ recheck_count,
                                                             const int* __restrict__ recheck_list,
                                                             int32_t* __restrict__ topk_idx, float* __restrict__ topk_w) {
  const int n = *recheck_count;
  const int lane = threadIdx.x & 63;
  for (int i = blockIdx.x * 4 + (threadIdx.x >> 6); i < n; i += gridDim.x * 4) {
    const int t = recheck_list[i];
    double zz[4], key[4], score[4];
    bool valid[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int e = lane + 64 * j;
      valid[j] = e < E;
      zz[j] = valid[j] ? z64[(size_t)i * E + e] : -__builtin_inf();
    }
    if (GATE == MOE_GATE_SOFTMAX) {
      double m = -__builtin_inf();
#pragma unroll
      for (int j = 0; j < 4; ++j) m = fmax(m, zz[j]);
#pragma unroll
      for (int o = 32; o > 0; o >>= 1) m = fmax(m, __shfl_xor(m, o, 64));
      double p[4], s = 0.0;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        p[j] = valid[j] ? exp(zz[j] - m) : 0.0;
        s += p[j];
      }
      s = wave_sum(s);
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        score[j] = p[j] / s;
        key[j] = zz[j];
      }
    } else {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int e = lane + 64 * j;
        score[j] = valid[j] ? 1.0 / (1.0 + exp(-zz[j])) : 0.0;
        key[j] = score[j] + ((bias && valid[j]) ? (double)bias[e] : 0.0);
      }
    }
    if (G > 0) group_limit_wave<double>(key, valid, E, G, M, lane);
    // K rounds of (key descending, index ascending) argmax over 64-bit ordered keys
    uint64_t ok[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) ok[j] = valid[j] ? f64_order(key[j]) : 0;
    int my_e = -1;
    for (int r = 0; r < K; ++r) {
      uint64_t best = 0;
      int best_e = 0x7FFFFFFF;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int e = lane + 64 * j;
        if (ok[j] > best || (ok[j] == best && ok[j] != 0 && e < best_e)) {
          best = ok[j];
          best_e = e;
        }
      }
#pragma unroll
      for (int o = 32; o > 0; o >>= 1) {
        const uint64_t ob = __shfl_xor(best, o, 64);
        const int oe = __shfl_xor(best_e, o, 64);
        if (ob > best || (ob == best && oe < best_e)) {
          best = ob;
          best_e = oe;
        }
      }
      if ((best_e & 63) == lane) {
#pragma unroll
        for (int j = 0; j < 4; ++j)
          if (j == (best_e >> 6)) ok[j] = 0;
      }
      if (lane == r) my_e = best_e;
    }
    const int src = my_e < 0 ? 0 : (my_e & 63);
    double g = 0.0;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const double v = __shfl(score[j], src, 64);
      if (my_e >= 0 && j == (my_e >> 6)) g = v;
    }
    if (renorm) g = g / wave_sum(lane < K ? g : 0.0);
    int rank = 0;
    for (int q = 0; q < K; ++q) rank += (__shfl(my_e, q, 64) < my_e) ? 1 : 0;
    if (lane < K) {
      topk_idx[(size_t)t * K + rank] = my_e;
      topk_w[(size_t)t * K + rank] = (float)g;
    }
  }
}

// ------------------------------------------------------------------ launchers
hipError_t launch_router_logits(const RouteArgs& a, hipStream_t s) {
  if (a.T == 0) return hipSuccess;
  if (a.u_bf16 && a.use_mfma) {
    launch_router_logits_mfma(a, s);
    return hipGetLastError();
  }
  const bool split = a.ksplit > 1;
  const int klen = split ? a.klen : a.d;
  double* zp = split ? a.zpart : nullptr;
  dim3 g1(cdiv(a.T, 64), cdiv(a.E, 64), split ? a.ksplit : 1);
  if (a.u_bf16)
    router_logits_valu<uint16_t><<<g1, 256, 0, s>>>((const uint16_t*)a.u, a.wg, a.off, a.T, a.E, a.d, klen, a.z, zp,
                                                    a.recheck_count, a.un2);
  else
    router_logits_valu<float><<<g1, 256, 0, s>>>((const float*)a.u, a.wg, a.off, a.T, a.E, a.d, klen, a.z, zp,
                                                 a.recheck_count, a.un2);
  if (split) {
    const long long n = (long long)a.T * a.E;
    const long long nb = (n + 255) / 256;
    router_logits_sum<<<(unsigned)(nb < 2048 ? nb : 2048), 256, 0, s>>>(a.zpart, a.ksplit, a.T, a.E, a.off, a.z);
  }
  return hipGetLastError();
}

hipError_t launch_route(const RouteArgs& a, hipStream_t s) {
  if (a.T == 0) return hipSuccess;
  hipError_t err = launch_router_logits(a, s);
  if (err != hipSuccess) return err;
  const int nb = cdiv(a.T, 4);
  // the logits kernels left the token norms per slice of d; the MFMA path also the centroid norms
  const bool mfma = a.u_bf16 && a.use_mfma;
  if (!mfma) router_prep_wg<false><<<a.E, 256, 0, s>>>(a.wg, a.E, a.d, a.wn2, nullptr);
  const int nsl = mfma ? router_mfma_slices(a.T, a.E, a.d) : a.ksplit;
  if (a.gate == MOE_GATE_SOFTMAX)
    router_topk<MOE_GATE_SOFTMAX><<<nb, 256, 0, s>>>(a.z, a.T, a.E, a.K, a.bias, a.renorm, a.n_groups, a.topk_groups,
                                                      a.delta, a.d, a.un2, nsl, a.wn2, a.topk_idx, a.topk_w,
                                                      a.recheck_count, a.recheck_list);
  else
    router_topk<MOE_GATE_SIGMOID_BIAS><<<nb, 256, 0, s>>>(a.z, a.T, a.E, a.K, a.bias, a.renorm, a.n_groups,
                                                           a.topk_groups, a.delta, a.d, a.un2, nsl, a.wn2, a.topk_idx,
                                                           a.topk_w, a.recheck_count, a.recheck_list);
  if (a.u_bf16)
    router_recheck_logits<uint16_t><<<dim3(a.E, kRecheckSplit), kRecheckThreads, 0, s>>>((const uint16_t*)a.u, a.wg, a.off, a.E, a.d,
                                                                     a.recheck_count, a.recheck_list, a.z64);
  else
    router_recheck_logits<float><<<dim3(a.E, kRecheckSplit), kRecheckThreads, 0, s>>>((const float*)a.u, a.wg, a.off, a.E, a.d,
                                                                  a.recheck_count, a.recheck_list, a.z64);
  if (a.gate == MOE_GATE_SOFTMAX)
    router_recheck_select<MOE_GATE_SOFTMAX><<<64, 256, 0, s>>>(a.z64, a.E, a.K, a.bias, a.renorm, a.n_groups,
                                                               a.topk_groups, a.recheck_count,
                                                               a.recheck_list, a.topk_idx, a.topk_w);
  else
    router_recheck_select<MOE_GATE_SIGMOID_BIAS><<<64, 256, 0, s>>>(a.z64, a.E, a.K, a.bias, a.renorm, a.n_groups,
                                                                    a.topk_groups,
                                                                    a.recheck_count, a.recheck_list, a.topk_idx,
                                                                    a.topk_w);
  return hipGetLastError();
}

}  // namespace moe
