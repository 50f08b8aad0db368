// Internal kernel launch interfaces of libmoe (not part of the C ABI).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

struct RouteArgs {
  const void* u;
  bool u_bf16;
  bool use_mfma;
  const float* wg;
  const float* off;
  const float* bias;
  int T, E, d, K, gate, renorm;
  int n_groups, topk_groups;   // group-limited routing (0: none)
  float delta;            // base recheck margin (scaled per token by the size of its partial sums)
  float* wn2;             // [E] squared centroid norms (scratch)
  float* un2;             // [slices, T] squared token norms per slice of d, written by the logits (scratch)
  float* z;               // [T, E] fp32 logits
  double* z64;            // [T, E] fp64 logits of rechecked tokens (compacted); MFMA logits: first the
                          // fp32 partial sums of up to four slices of d ([T, E] x 16 bytes)
  uint16_t* wg_split;     // [3, E, d] bf16 parts of w_gate (MFMA logits)
  double* zpart;          // [ksplit, T, E] fp64 partial logits over slices of d (vector-ALU logits)
  int ksplit, klen;       // slices of d and their length (a multiple of 32); ksplit 1 writes z directly
  int* recheck_count;
  int* recheck_list;      // [T]
  int32_t* topk_idx;
  float* topk_w;
};

// Block shape of the MFMA router logits: 256 tokens x 128 experts when four slices of d give at least one
// block per CU of the chip's 256, else 128 tokens x 64 experts.
inline bool router_mfma_large(int T, int E) {
  return (long long)((T + 255) / 256) * ((E + 127) / 128) * 4 >= 256;
}

// Slices of d for the MFMA router logits, at most four, each at least 8 stages of 64: for the small
// blocks enough for about 512 (two per CU; at the V3 shape with them, 256 blocks: two slices, three
// measured slower), for the large ones about 256 (one per CU: 8 waves).
inline int router_mfma_slices(int T, int E, int d) {
  const bool large = router_mfma_large(T, E);
  const long long blocks = large ? (long long)((T + 255) / 256) * ((E + 127) / 128)
                                 : (long long)((T + 127) / 128) * ((E + 63) / 64);
  if (blocks <= 0) return 1;
  long long ks = (large ? 256 : 512) / blocks;
  ks = ks < 1 ? 1 : (ks > 4 ? 4 : ks);
  while (ks > 1 && d / 64 < 8 * ks) --ks;
  return (int)ks;
}

// Slices of d for the vector-ALU router logits: enough 64x64 blocks to cover the chip when T and E are
// small (a decode step), each slice at least 128 long, partial sums at most 64 MiB. Sets klen.
inline int router_ksplit(int T, int E, int d, int& klen) {
  const long long blocks = (long long)((T + 63) / 64) * ((E + 63) / 64);
  if (blocks <= 0 || d <= 0) {   // no tokens: nothing to split
    klen = d;
    return 1;
  }
  long long s = (512 + blocks - 1) / blocks;
  s = s < 1 ? 1 : s;
  const long long smax = (d + 127) / 128;
  s = s > smax ? smax : s;
  while (s > 1 && s * T * (long long)E * 8 > (64LL << 20)) s /= 2;
  const int per = (int)((d + s - 1) / s);
  klen = (per + 31) / 32 * 32;
  return (d + klen - 1) / klen;
}

struct DispatchArgs {
  const int32_t* topk_idx;
  int T, E, K;
  int32_t* chunk_counts;  // [chunks, E]
  int32_t* counts;
  int32_t* offsets;
  int32_t* perm_src;
  int32_t* row_of;
};

// Load-balance statistics of one routed batch.
struct BalanceArgs {
  const float* z;         // [T, E] router logits
  const int32_t* idx;     // [T, K] selected experts
  int T, E, K, gate, seq_len;
  float alpha_expert, alpha_seq;
  double* psum;           // [chunks, E] per-chunk sums of routing probabilities
  int32_t* cnt;           // [chunks, E] per-chunk selection counts
  double* seq_p;          // [T / seq_len, E] per-sequence sums of routing probabilities
  int32_t* seq_n;         // [T / seq_len, E] per-sequence selection counts
  double* seq_term;       // [T / seq_len] sum_i f_i P_i of each sequence
  float* f;               // [E] out
  float* P;               // [E] out
  float* loss;            // [2] out: expert-level, sequence-wise
};

// One grouped GEMM launch (gate/up + SwiGLU, or down) over the E routed groups and the shared group.
struct GemmArgs {
  int E, T, d, f, fs;
  const int32_t* offsets;
  const int32_t* perm_src;
  const int32_t* mt_prefix;   // [E+1] prefix of M tiles per routed expert
  const int32_t* xrange;      // matrix-core path: [kSchedRange] tile-id ranges (see launch_schedule_mfma)
  int32_t* xcount;            // matrix-core path: [kSchedCount] tile counters, zero at launch
  const uint8_t* w_routed;    // w13 or w2 of all routed experts
  const uint8_t* w_shared;
  const float* ws_routed;     // fp8 block scales
  const float* ws_shared;
  const uint8_t* x_routed;    // gate/up: u (gathered through perm_src); down: a rows
  const uint8_t* x_shared;
  const float* xs_routed;     // fp8 activation scales
  const float* xs_shared;
  uint8_t* out_routed;        // gate/up: a; down: y
  uint8_t* out_shared;
  float* out_scale_routed;    // gate/up fp8: scales of a
  float* out_scale_shared;
  int packed;                 // weights in the tiled layout of launch_pack_weights (matrix-core kernels only)
  // Matrix-core kernels, E4M3: layout of the token scales. 0: [rows][kblk] (row r, block kb at r * kblk + kb);
  // ld > 0: [kblk][ld] (at kb * ld + r), so that one stage's scales of a tile's consecutive rows are contiguous.
  int xs_ld_routed, xs_ld_shared;
  int os_ld_routed, os_ld_shared;   // the same choice for the scales of a written by the gate/up epilogue
};

hipError_t launch_route(const RouteArgs& a, hipStream_t s);
hipError_t launch_router_logits(const RouteArgs& a, hipStream_t s);
void launch_router_logits_mfma(const RouteArgs& a, hipStream_t s);
hipError_t launch_dispatch(const DispatchArgs& a, hipStream_t s);
int dispatch_chunks(int T);
hipError_t launch_quant_act(const void* x, bool x_bf16, int rows, int cols, uint8_t* q, float* scales, hipStream_t s);
// out[kb * ld + r] = xs[src(r) * kblk + kb] for r < n, src(r) = perm[r] (perm non-null; n = *n_rows, the
// dispatched row count, at most rows) or r (perm null; n = rows): the 1x128 scales of gathered rows, block-major.
// The same launch also writes out2[kb * ld2 + r] = xs[r * kblk + kb] for r < rows2 (rows2 = 0: nothing).
hipError_t launch_scales_by_block(const float* xs, int kblk, const int32_t* perm, const int32_t* n_rows, int rows,
                                  float* out, int ld, int rows2, float* out2, int ld2, hipStream_t s);
hipError_t launch_quant_weight(const float* w, int batch, int rows, int cols, uint8_t* q, float* scales, hipStream_t s);
hipError_t launch_schedule(const int32_t* offsets, int E, int bm, int32_t* mt_prefix, hipStream_t s);
// M-tile prefix plus, for the gate/up (k = 0) and down (k = 1) launches of the matrix-core GEMM, the
// tile ranges xrange[k][kSchedRange] and zeroed tile counters xcount[k][kSchedCount]: tiles
// [xrange[x], xrange[x + 1]) belong to XCD x (x < 8, equal estimated cost), [xrange[8], xrange[9]) are a
// pool that any block takes from once its XCD's range is done (counter 8; the last 1/kSchedPoolDiv of
// the cost), so that blocks of every XCD finish together.
constexpr int kSchedRange = 10, kSchedCount = 9, kSchedPoolDiv = 8;
hipError_t launch_schedule_mfma(const int32_t* offsets, int E, int T, int bm, const int (&nt_r)[2], const int (&nt_s)[2],
                                int32_t* mt_prefix, int32_t* xrange, int32_t* xcount, hipStream_t s);
// The tile schedule's arguments (as launch_schedule_mfma), for launches that compute it beside other work.
struct SchedArgs {
  const int32_t* offsets;
  int E, T, bm;
  int nt_r[2], nt_s[2];
  int32_t* mt_prefix;
  int32_t* xrange;
  int32_t* xcount;
};
// launch_quant_act (bf16 x) and launch_schedule_mfma in one launch
hipError_t launch_quant_act_schedule(const void* x, int rows, int cols, uint8_t* q, float* scales, const SchedArgs& sa,
                                     hipStream_t s);
int gemm_mfma_bm();
// raw (E4M3 only): fp32 accumulators out (gate/up: g and v without SwiGLU; down: fp32 instead of bf16)
hipError_t launch_gemm_mfma(const GemmArgs& a, bool fp8, bool gateup, int grid, hipStream_t s, bool raw = false);
// weights of `groups` groups of [rows, row_bytes] (row-major, one group after the other) -> the tiled
// layout the matrix-core and decode kernels read with GemmArgs::packed (gateup: rows = 2 x inner dim,
// W1 rows then W3 rows; else W2 rows); rows % 256 == 0, row_bytes % 128 == 0
hipError_t launch_pack_weights(const void* src, void* dst, int groups, int rows, int row_bytes, bool gateup,
                               hipStream_t s);
hipError_t launch_swiglu_backward_quant(const float* da, const float* gv, int rows, int fg, uint8_t* q, float* scales,
                                        hipStream_t s);
hipError_t launch_transpose_fp8(const uint8_t* q, const float* scales, int batch, int rows, int cols, uint8_t* qt,
                                float* scales_t, hipStream_t s);
// Weight gradients of the E4M3 experts: row-block prefix, quantization along the rows (transposed
// out), and the grouped row-scaled GEMM.
enum { kWgSrcDy = 0, kWgSrcX = 1, kWgSrcA = 2, kWgSrcDgv = 3 };
struct WgQuantArgs {
  const int32_t* offsets;     // [E+1] routed row offsets
  const int32_t* perm;        // [T*K] token of each routed row (source X)
  const int32_t* pblk;        // [E+2] row-block prefix (routed experts, then the shared block)
  int E, T, C, fg;            // C channels of the operand; fg inner dim of [g | v] and da
  const uint16_t* bf_r;       // DY: dy_routed [T*K][C]; X: u [T][C]
  const uint16_t* bf_s;       // DY: dy_shared [T][C]; X: u
  const float* gv_r;          // A, DGV: [g | v] rows [.][2 fg]
  const float* gv_s;
  const float* da_r;          // DGV: da rows [.][fg]
  const float* da_s;
  uint8_t* qt;                // codes [C][rpad]
  float* st;                  // scales [row block][C]
  size_t rpad;                // padded rows of qt (row stride)
};
struct WgGemmArgs {
  const int32_t* pblk;
  int32_t* xcount;            // 9 tile counters (one per XCD, then the pool's), zero at launch
  int E, shared, M, N;        // output [M][N] per group (multiples of 128)
  const uint8_t* A;           // [N][rpad] codes, scales As [row block][N]
  const float* As;
  const uint8_t* B;           // [M][rpad] codes, scales Bs [row block][M]
  const float* Bs;
  size_t rpad;
  uint16_t* out_r;            // bf16 [E][M][N]
  uint16_t* out_s;            // bf16 [M][N]
};
int wgrad_row_blocks_max(int T, int K, int E, bool shared);
// pblk[0..E+1], then 18 zeroed tile counters (two launches of the weight-gradient GEMM)
hipError_t launch_wgrad_prefix(const int32_t* offsets, int E, int T, bool shared, int32_t* pblk, hipStream_t s);
hipError_t launch_wgrad_quant(const WgQuantArgs& a, int src, int nblk_max, hipStream_t s);
hipError_t launch_wgrad_gemm(const WgGemmArgs& a, int grid, hipStream_t s);   // grid >= 8 (one block per CU)
int balance_chunks_for(int T);
int balance_sequences_max(int T);   // sequences of T tokens when seq_len is T or a multiple of 64
hipError_t launch_balance_stats(const BalanceArgs& a, hipStream_t s);
// E4M3 grouped GEMMs for batches of at most gemm_decode_max_tokens() tokens (weight streaming)
int gemm_decode_max_tokens();
hipError_t launch_gemm_decode(const GemmArgs& a, bool gateup, hipStream_t s);
int gemm_simt_bm();
hipError_t launch_gemm_simt(const GemmArgs& a, bool gateup, int max_tiles, hipStream_t s);
hipError_t launch_combine(const void* u, bool bf16, const void* y_routed, const void* y_shared, bool y_bf16,
                          const int32_t* row_of, const float* topk_w, int T, int d, int K, void* h, hipStream_t s);
hipError_t launch_zero_fill(void* p, size_t bytes, hipStream_t s);
hipError_t launch_bias_update(const int32_t* counts, int E, long long TK, float gamma, float* bias, hipStream_t s);

}  // namespace moe
