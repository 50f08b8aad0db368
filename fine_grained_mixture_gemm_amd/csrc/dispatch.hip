// Dispatch: expert histogram, prefix sums and the stable permutation of (token, slot) pairs into
// expert-contiguous rows.
//
// Tokens are processed in chunks of 256 (one per thread). In LDS each chunk builds one bit per
// (expert, token): the chunk's count of an expert is a popcount, and a token's rank among the chunk's
// tokens of that expert is the popcount of the bits below it, so rows come out in ascending token
// order without any ordering of atomics.
#include "common.h"
#include "kernels.h"

namespace moe {

constexpr int kChunk = 256;
constexpr int kWords = kChunk / 32;

// A (token, slot) pair enters the permutation when its id names a routed expert and no earlier slot of
// the token holds the same id: one row per (token, expert). Other pairs are dropped (row_of = -1).
__device__ __forceinline__ bool pair_kept(const int32_t* __restrict__ ids, int k, int E) {
  const int e = ids[k];
  if (e < 0 || e >= E) return false;
  for (int j = 0; j < k; ++j)
    if (ids[j] == e) return false;
  return true;
}

__device__ __forceinline__ void build_bits(uint32_t (*bits)[kWords], const int32_t* __restrict__ idx, int T, int E,
                                           int K, int c) {
  for (int i = threadIdx.x; i < E * kWords; i += blockDim.x) (&bits[0][0])[i] = 0u;
  __syncthreads();
  const int tl = threadIdx.x, t = c * kChunk + tl;
  if (t < T) {
    for (int k = 0; k < K; ++k) {
      const int e = idx[(size_t)t * K + k];
      if (pair_kept(idx + (size_t)t * K, k, E)) atomicOr(&bits[e][tl >> 5], 1u << (tl & 31));
    }
  }
  __syncthreads();
}

__global__ __launch_bounds__(kChunk) void dispatch_count(const int32_t* __restrict__ idx, int T, int E, int K,
                                                         int32_t* __restrict__ chunk_counts) {
  __shared__ uint32_t bits[256][kWords];
  const int c = blockIdx.x;
  build_bits(bits, idx, T, E, K, c);
  for (int e = threadIdx.x; e < E; e += blockDim.x) {
    int n = 0;
#pragma unroll
    for (int w = 0; w < kWords; ++w) n += __popc(bits[e][w]);
    chunk_counts[(size_t)c * E + e] = n;
  }
}

// One block: per-expert running sums over chunks, expert counts and offsets.
__global__ __launch_bounds__(256) void dispatch_scan(const int32_t* __restrict__ chunk_counts, int nchunks, int E,
                                                     int32_t* __restrict__ chunk_base, int32_t* __restrict__ counts,
                                                     int32_t* __restrict__ offsets) {
  __shared__ int32_t s_cnt[256];
  const int e = threadIdx.x;
  int run = 0;
  if (e < E) {
    for (int c = 0; c < nchunks; ++c) {
      chunk_base[(size_t)c * E + e] = run;
      run += chunk_counts[(size_t)c * E + e];
    }
    counts[e] = run;
  }
  s_cnt[e] = e < E ? run : 0;
  __syncthreads();
  if (e == 0) {
    int o = 0;
    for (int i = 0; i < E; ++i) {
      offsets[i] = o;
      o += s_cnt[i];
    }
    offsets[E] = o;
  }
}

__global__ __launch_bounds__(kChunk) void dispatch_scatter(const int32_t* __restrict__ idx, int T, int E, int K,
                                                           const int32_t* __restrict__ chunk_base,
                                                           const int32_t* __restrict__ offsets,
                                                           int32_t* __restrict__ perm_src, int32_t* __restrict__ row_of) {
  __shared__ uint32_t bits[256][kWords];
  const int c = blockIdx.x;
  build_bits(bits, idx, T, E, K, c);
  const int tl = threadIdx.x, t = c * kChunk + tl;
  if (t >= T) return;
  const int w0 = tl >> 5;
  const uint32_t below = (1u << (tl & 31)) - 1u;
  for (int k = 0; k < K; ++k) {
    const int e = idx[(size_t)t * K + k];
    if (!pair_kept(idx + (size_t)t * K, k, E)) {
      row_of[(size_t)t * K + k] = -1;
      continue;
    }
    int rank = __popc(bits[e][w0] & below);
    for (int w = 0; w < w0; ++w) rank += __popc(bits[e][w]);
    const int row = offsets[e] + chunk_base[(size_t)c * E + e] + rank;
    perm_src[row] = t;
    row_of[(size_t)t * K + k] = row;
  }
}

hipError_t launch_dispatch(const DispatchArgs& a, hipStream_t s) {
  if (a.T == 0) return hipSuccess;
  const int nchunks = cdiv(a.T, kChunk);
  dispatch_count<<<nchunks, kChunk, 0, s>>>(a.topk_idx, a.T, a.E, a.K, a.chunk_counts);
  dispatch_scan<<<1, 256, 0, s>>>(a.chunk_counts, nchunks, a.E, a.chunk_base, a.counts, a.offsets);
  dispatch_scatter<<<nchunks, kChunk, 0, s>>>(a.topk_idx, a.T, a.E, a.K, a.chunk_base, a.offsets, a.perm_src, a.row_of);
  return hipGetLastError();
}

int dispatch_chunks(int T) { return cdiv(T, kChunk); }

}  // namespace moe
