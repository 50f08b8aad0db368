// Load-balance statistics of one routed batch.
//
// DeepSeek Technical Report: MoE Architecture, 1.2: the expert-level balance loss
// L_ExpBal = alpha_1 sum_i f_i P_i, f_i the fraction of tokens that selected expert i, P_i the average
// routing probability of expert i (alpha_1 = 0.003 in 2.3); 3.3: V3 adds a sequence-wise balance loss of
// very small weight, whose formula the report does not print. Here: f_i = count_i / T (no E/K
// normalisation is printed), P_i = mean over tokens of the probability over all routed experts (softmax
// of the logits, or sigmoid affinities normalised over all routed experts), and the sequence-wise loss is
// alpha_seq times the mean over sequences of sum_i f_i^b P_i^b computed within each sequence.
//
// Three deterministic passes (fp64 sums in a fixed order, no atomics):
//   1. one block per 16-token chunk: per-expert sums of the routing probabilities and selection counts;
//   2. one block per sequence: its chunks summed in a fixed order, per-sequence totals, sum_i f_i^b P_i^b;
//   3. one block: batch f, P (from the sequence totals) and both losses.
#include "common.h"
#include "kernels.h"

namespace moe {

constexpr int kBalChunk = 16;    // tokens per chunk (a sequence is T or a multiple of 64 tokens, so chunks
                                 // never straddle one)
constexpr int kBalThreads = 256;

// Tree sum of one fp64 value per thread of a 256-thread block, in a fixed order (buf: 256 doubles).
__device__ __forceinline__ double block_sum_fixed(double v, double* buf) {
  const int t = threadIdx.x;
  buf[t] = v;
  __syncthreads();
  for (int o = kBalThreads / 2; o > 0; o >>= 1) {
    if (t < o) buf[t] += buf[t + o];
    __syncthreads();
  }
  const double r = buf[0];
  __syncthreads();
  return r;
}

// Pass 1. Wave w of the block takes tokens chunk_start + w, + 4, ...; a lane holds experts lane + 64 q.
template <int GATE>
__global__ __launch_bounds__(kBalThreads) void balance_chunks(const float* __restrict__ z,
                                                              const int32_t* __restrict__ idx, int T, int E, int K,
                                                              double* __restrict__ psum, int32_t* __restrict__ cnt) {
  __shared__ double s_p[4][256];
  __shared__ int32_t s_c[4][256];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int t0 = blockIdx.x * kBalChunk, t1 = min(T, t0 + kBalChunk);
  double acc[4] = {0.0, 0.0, 0.0, 0.0};
  int c[4] = {0, 0, 0, 0};
  for (int t = t0 + wave; t < t1; t += 4) {
    double v[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int e = lane + 64 * q;
      v[q] = e < E ? (double)z[(size_t)t * E + e] : 0.0;
    }
    double p[4];
    if (GATE == MOE_GATE_SOFTMAX) {
      double m = -INFINITY;
#pragma unroll
      for (int q = 0; q < 4; ++q)
        if (lane + 64 * q < E) m = fmax(m, v[q]);
      for (int o = 32; o > 0; o >>= 1) m = fmax(m, __shfl_xor(m, o, 64));
#pragma unroll
      for (int q = 0; q < 4; ++q) p[q] = lane + 64 * q < E ? exp(v[q] - m) : 0.0;
    } else {
#pragma unroll
      for (int q = 0; q < 4; ++q) p[q] = lane + 64 * q < E ? 1.0 / (1.0 + exp(-v[q])) : 0.0;
    }
    const double sum = wave_sum((p[0] + p[1]) + (p[2] + p[3]));
#pragma unroll
    for (int q = 0; q < 4; ++q) acc[q] += p[q] / sum;
    for (int k = 0; k < K; ++k) {
      const int e = idx[(size_t)t * K + k];
#pragma unroll
      for (int q = 0; q < 4; ++q) c[q] += e == lane + 64 * q ? 1 : 0;
    }
  }
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    s_p[wave][lane + 64 * q] = acc[q];
    s_c[wave][lane + 64 * q] = c[q];
  }
  __syncthreads();
  const int e = threadIdx.x;
  if (e < E) {
    psum[(size_t)blockIdx.x * E + e] = (s_p[0][e] + s_p[1][e]) + (s_p[2][e] + s_p[3][e]);
    cnt[(size_t)blockIdx.x * E + e] = s_c[0][e] + s_c[1][e] + s_c[2][e] + s_c[3][e];
  }
}

// Pass 2. Block b (1024 threads: expert e = tid % 256, lane r = tid / 256) sums the chunks of sequence b:
// lane r takes chunks r, r + 4, ..., the four partial sums are added in lane order. Writes the sequence's
// per-expert totals and sum_e f_e^b P_e^b.
__global__ __launch_bounds__(1024) void balance_sequences(const double* __restrict__ psum,
                                                         const int32_t* __restrict__ cnt, int E, int chunks_per_seq,
                                                         int seq_len, double* __restrict__ seq_p,
                                                         int32_t* __restrict__ seq_n, double* __restrict__ seq_term) {
  __shared__ double sp[4][256];
  __shared__ int32_t sn[4][256];
  __shared__ double buf[kBalThreads];
  const int e = threadIdx.x & 255, r = threadIdx.x >> 8;
  double p = 0.0;
  int n = 0;
  if (e < E) {
    for (int k = r; k < chunks_per_seq; k += 4) {
      const size_t ch = (size_t)blockIdx.x * chunks_per_seq + k;
      p += psum[ch * E + e];
      n += cnt[ch * E + e];
    }
  }
  sp[r][e] = p;
  sn[r][e] = n;
  __syncthreads();
  if (r == 0) {
    double fp = 0.0;
    if (e < E) {
      const double pt = (sp[0][e] + sp[1][e]) + (sp[2][e] + sp[3][e]);
      const int nt = sn[0][e] + sn[1][e] + sn[2][e] + sn[3][e];
      seq_p[(size_t)blockIdx.x * E + e] = pt;
      seq_n[(size_t)blockIdx.x * E + e] = nt;
      fp = ((double)nt / seq_len) * (pt / seq_len);
    }
    buf[e] = fp;
  }
  __syncthreads();
  for (int o = kBalThreads / 2; o > 0; o >>= 1) {
    if (threadIdx.x < o) buf[threadIdx.x] += buf[threadIdx.x + o];
    __syncthreads();
  }
  if (threadIdx.x == 0) seq_term[blockIdx.x] = buf[0];
}

// Pass 3. Batch f_e = count_e / T, P_e = sum_e / T from the sequence totals (in sequence order),
// L_ExpBal = alpha_expert sum f P, L_seq = alpha_seq * mean of the sequence terms.
__global__ __launch_bounds__(kBalThreads) void balance_finish(const double* __restrict__ seq_p,
                                                              const int32_t* __restrict__ seq_n,
                                                              const double* __restrict__ seq_term, int E, int T,
                                                              int n_seq, float alpha_expert, float alpha_seq,
                                                              float* __restrict__ f, float* __restrict__ P,
                                                              float* __restrict__ loss) {
  __shared__ double buf[kBalThreads];
  const int e = threadIdx.x;
  double fe = 0.0, pe = 0.0;
  if (e < E) {
    double p = 0.0;
    long long n = 0;
    for (int b = 0; b < n_seq; ++b) {
      p += seq_p[(size_t)b * E + e];
      n += seq_n[(size_t)b * E + e];
    }
    fe = (double)n / T;
    pe = p / T;
    f[e] = (float)fe;
    P[e] = (float)pe;
  }
  const double fp = block_sum_fixed(fe * pe, buf);
  if (e == 0) {
    double s = 0.0;
    for (int b = 0; b < n_seq; ++b) s += seq_term[b];
    loss[0] = (float)((double)alpha_expert * fp);
    loss[1] = (float)((double)alpha_seq * (s / n_seq));
  }
}

int balance_chunks_for(int T) { return cdiv(T, kBalChunk); }
int balance_sequences_max(int T) { return cdiv(T, 64); }

hipError_t launch_balance_stats(const BalanceArgs& a, hipStream_t s) {
  if (a.T == 0) return hipSuccess;
  const int chunks = cdiv(a.T, kBalChunk);
  const int n_seq = a.T / a.seq_len;
  const int cps = cdiv(a.seq_len, kBalChunk);
  if (a.gate == MOE_GATE_SOFTMAX)
    balance_chunks<MOE_GATE_SOFTMAX><<<chunks, kBalThreads, 0, s>>>(a.z, a.idx, a.T, a.E, a.K, a.psum, a.cnt);
  else
    balance_chunks<MOE_GATE_SIGMOID_BIAS><<<chunks, kBalThreads, 0, s>>>(a.z, a.idx, a.T, a.E, a.K, a.psum, a.cnt);
  balance_sequences<<<n_seq, 1024, 0, s>>>(a.psum, a.cnt, a.E, cps, a.seq_len, a.seq_p, a.seq_n, a.seq_term);
  balance_finish<<<1, kBalThreads, 0, s>>>(a.seq_p, a.seq_n, a.seq_term, a.E, a.T, n_seq, a.alpha_expert,
                                           a.alpha_seq, a.f, a.P, a.loss);
  return hipGetLastError();
}

}  // namespace moe
