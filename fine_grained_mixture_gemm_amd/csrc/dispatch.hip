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
// The token's K <= 16 ids are held in registers.
__device__ __forceinline__ bool pair_kept(const int (&ids)[16], int k, int E) {
  const int e = ids[k];
  if (e < 0 || e >= E) return false;
  for (int j = 0; j < k; ++j)
    if (ids[j] == e) return false;
  return true;
}

__device__ __forceinline__ void load_ids(const int32_t* __restrict__ idx, int t, int T, int K, int (&ids)[16]) {
#pragma unroll
  for (int k = 0; k < 16; ++k) ids[k] = (t < T && k < K) ? idx[(size_t)t * K + k] : -1;
}

__device__ __forceinline__ void build_bits(uint32_t (*bits)[kWords], const int (&ids)[16], int t, int T, int E, int K) {
  for (int i = threadIdx.x; i < E * kWords; i += blockDim.x) (&bits[0][0])[i] = 0u;
  __syncthreads();
  const int tl = threadIdx.x;
  if (t < T) {
    for (int k = 0; k < K; ++k)
      if (pair_kept(ids, k, E)) atomicOr(&bits[ids[k]][tl >> 5], 1u << (tl & 31));
  }
  __syncthreads();
}

// exclusive prefix sum of v over the block's 256 threads, and the total
__device__ __forceinline__ int block_exclusive_scan_256(int v, int* s_wave, int& total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  int x = v;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int y = __shfl_up(x, o, 64);
    if (lane >= o) x += y;
  }
  if (lane == 63) s_wave[wave] = x;
  __syncthreads();
  int before = 0;
  total = 0;
#pragma unroll
  for (int w = 0; w < kChunk / 64; ++w) {
    const int tw = s_wave[w];
    if (w < wave) before += tw;
    total += tw;
  }
  return before + x - v;
}

// Rows of the chunk's kept pairs: base[e] (first row of expert e for this chunk) plus the pair's rank
// among the chunk's tokens of expert e.
__device__ __forceinline__ void scatter_rows(const uint32_t (*bits)[kWords], const int32_t* base, const int (&ids)[16],
                                             int t, int T, int E, int K, int32_t* __restrict__ perm_src,
                                             int32_t* __restrict__ row_of) {
  if (t >= T) return;
  const int tl = threadIdx.x, w0 = tl >> 5;
  const uint32_t below = (1u << (tl & 31)) - 1u;
  for (int k = 0; k < K; ++k) {
    if (!pair_kept(ids, k, E)) {
      row_of[(size_t)t * K + k] = -1;
      continue;
    }
    const int e = ids[k];
    int rank = __popc(bits[e][w0] & below);
    for (int w = 0; w < w0; ++w) rank += __popc(bits[e][w]);
    const int row = base[e] + rank;
    perm_src[row] = t;
    row_of[(size_t)t * K + k] = row;
  }
}

__global__ __launch_bounds__(kChunk) void dispatch_count(const int32_t* __restrict__ idx, int T, int E, int K,
                                                         int32_t* __restrict__ chunk_counts) {
  __shared__ uint32_t bits[256][kWords];
  const int c = blockIdx.x, t = c * kChunk + threadIdx.x;
  int ids[16];
  load_ids(idx, t, T, K, ids);
  build_bits(bits, ids, t, T, E, K);
  for (int e = threadIdx.x; e < E; e += blockDim.x) {
    int n = 0;
#pragma unroll
    for (int w = 0; w < kWords; ++w) n += __popc(bits[e][w]);
    chunk_counts[(size_t)c * E + e] = n;
  }
}

// Every block first reads all chunks' counts (E x chunks values, from L2): thread e sums expert e's
// counts over the chunks before this one (its rows come after theirs) and over all chunks (the expert's
// count), and a block-wide scan of the counts gives the experts' first rows. Block 0 also writes counts
// and offsets. This replaces a separate scan launch between the two passes.
__global__ __launch_bounds__(kChunk) void dispatch_scatter(const int32_t* __restrict__ idx, int T, int E, int K,
                                                           const int32_t* __restrict__ chunk_counts, int nchunks,
                                                           int32_t* __restrict__ counts, int32_t* __restrict__ offsets,
                                                           int32_t* __restrict__ perm_src, int32_t* __restrict__ row_of) {
  __shared__ uint32_t bits[256][kWords];
  __shared__ int32_t base[256];
  __shared__ int s_wave[kChunk / 64];
  const int c = blockIdx.x, t = c * kChunk + threadIdx.x, e = threadIdx.x;
  int before = 0, total_e = 0;
  if (e < E) {
    for (int cc = 0; cc < nchunks; ++cc) {
      const int v = chunk_counts[(size_t)cc * E + e];
      before += cc < c ? v : 0;
      total_e += v;
    }
  }
  int total;
  const int off = block_exclusive_scan_256(e < E ? total_e : 0, s_wave, total);
  if (e < E) {
    base[e] = off + before;
    if (c == 0) {
      counts[e] = total_e;
      offsets[e] = off;
    }
  }
  if (c == 0 && e == 0) offsets[E] = total;
  int ids[16];
  load_ids(idx, t, T, K, ids);
  build_bits(bits, ids, t, T, E, K);   // its barriers also publish `base`
  scatter_rows(bits, base, ids, t, T, E, K, perm_src, row_of);
}

// T <= 256: the whole dispatch in one block (histogram, offsets and permutation).
__global__ __launch_bounds__(kChunk) void dispatch_single(const int32_t* __restrict__ idx, int T, int E, int K,
                                                          int32_t* __restrict__ counts, int32_t* __restrict__ offsets,
                                                          int32_t* __restrict__ perm_src, int32_t* __restrict__ row_of) {
  __shared__ uint32_t bits[256][kWords];
  __shared__ int32_t base[256];
  __shared__ int s_wave[kChunk / 64];
  const int t = threadIdx.x, e = threadIdx.x;
  int ids[16];
  load_ids(idx, t, T, K, ids);
  build_bits(bits, ids, t, T, E, K);
  int n = 0;
  if (e < E) {
#pragma unroll
    for (int w = 0; w < kWords; ++w) n += __popc(bits[e][w]);
  }
  int total;
  const int off = block_exclusive_scan_256(n, s_wave, total);
  if (e < E) {
    counts[e] = n;
    offsets[e] = off;
    base[e] = off;
  }
  if (e == 0) offsets[E] = total;
  __syncthreads();
  scatter_rows(bits, base, ids, t, T, E, K, perm_src, row_of);
}

hipError_t launch_dispatch(const DispatchArgs& a, hipStream_t s) {
  if (a.T == 0) return hipSuccess;
  if (a.T <= kChunk) {
    dispatch_single<<<1, kChunk, 0, s>>>(a.topk_idx, a.T, a.E, a.K, a.counts, a.offsets, a.perm_src, a.row_of);
    return hipGetLastError();
  }
  const int nchunks = cdiv(a.T, kChunk);
  dispatch_count<<<nchunks, kChunk, 0, s>>>(a.topk_idx, a.T, a.E, a.K, a.chunk_counts);
  dispatch_scatter<<<nchunks, kChunk, 0, s>>>(a.topk_idx, a.T, a.E, a.K, a.chunk_counts, nchunks, a.counts, a.offsets,
                                              a.perm_src, a.row_of);
  return hipGetLastError();
}

int dispatch_chunks(int T) { return cdiv(T, kChunk); }

}  // namespace moe
