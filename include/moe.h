/*
 * moe.h - C ABI of the DeepSeekMoE layer forward pass on one AMD Instinct MI355X (gfx950).
 *
 * The layer (DeepSeek Technical Report: MoE Architecture, 1.1 "Shared Expert Isolation" formula and
 * 5.3 [1]) computes, for every token t with input row u_t:
 *
 *     h_t = u_t + sum_{i <= Ks} FFN_i(u_t) + sum_{i in TopK(t)} g_{i,t} FFN_i(u_t)
 *
 * with fine-grained routed SwiGLU experts FFN(x) = W2 (SiLU(W1 x) * (W3 x)) (DeepSeek-V3 walkthrough,
 * "invariant core"), gates from a softmax over the routed experts (same report, 2.3) or from sigmoid
 * affinities whose selection key carries a per-expert bias that never enters the gate (same report,
 * 3.3 "Auxiliary-Loss-Free Load Balancing"), and optionally every expert GEMM in E4M3 with 1x128
 * activation tiles, 128x128 weight blocks and FP32 accumulation promoted every 128 elements (same
 * report, 3.6 "FP8 Mixed Precision Training").
 *
 * Conventions shared by every entry point:
 *  - Every pointer argument is a DEVICE pointer unless marked "host". The caller owns every buffer;
 *    the library allocates nothing. Scratch memory comes from a caller-provided workspace of at least
 *    moe_workspace_size() bytes, 256-byte aligned.
 *  - Device buffers of activations, weights, expert outputs and gradients must start on a 16-byte
 *    boundary (the kernels move them in 16-byte pieces); a misaligned one fails with
 *    MOE_ERR_INVALID_ARG. torch and hipMalloc allocations always satisfy this.
 *  - Calls validate their arguments synchronously (nothing is launched when they fail) and then enqueue
 *    work on `stream` asynchronously. They never abort and never synchronize the device.
 *  - Matrices are row-major. T = tokens, d = d_model, E = routed experts, Ks = shared experts,
 *    K = routed experts per token, f = routed expert inner dim, fs = Ks * f. The Ks shared experts are
 *    stored as one SwiGLU block of inner dim fs (concatenating the inner dims is the same as summing).
 *  - Activations u and the output h have dtype act_dtype (F32 or BF16, bf16 = raw uint16 bits).
 *  - Expert weights have dtype w_dtype. Supported (act, w) pairs: (F32, F32), (BF16, BF16),
 *    (BF16, FP8_E4M3). bf16 and fp8 weights need d % 256 == 0 and f % 128 == 0; d <= 8192.
 *  - Expert outputs y (per routed row and shared) are BF16 for FP8_E4M3 weights (the combine payload of
 *    the E4M3 design) and F32 otherwise.
 *  - On a non-OK status, moe_last_error() returns a message for the calling thread.
 */
#ifndef MOE_MI355X_H
#define MOE_MI355X_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  MOE_OK = 0,
  MOE_ERR_INVALID_ARG = 1,   /* null pointer, negative size, K > E, bad enum value */
  MOE_ERR_UNSUPPORTED = 2,   /* valid but not implemented: dtype pair, E > 256, K > 16, tile alignment */
  MOE_ERR_WORKSPACE = 3,     /* workspace missing or smaller than moe_workspace_size() */
  MOE_ERR_HIP = 4            /* a HIP launch or API call failed (message names it) */
} moe_status;

typedef enum { MOE_F32 = 0, MOE_BF16 = 1, MOE_FP8_E4M3 = 2 } moe_dtype;

/* Gating: softmax over the routed experts (DeepSeek Technical Report: MoE Architecture, 2.3), or
 * sigmoid affinity with the selection-only bias (same report, 3.3). */
typedef enum { MOE_GATE_SOFTMAX = 0, MOE_GATE_SIGMOID_BIAS = 1 } moe_gate;

/* Storage of the expert weight matrices of a layer (moe_layer.weight_layout). */
typedef enum {
  MOE_LAYOUT_ROWS = 0,   /* row-major, as documented at moe_layer */
  MOE_LAYOUT_TILED = 1   /* the tiled layout written by moe_pack_weights (bf16 and fp8 weights) */
} moe_weight_layout;

/* Which weight matrix moe_pack_weights converts. */
typedef enum {
  MOE_PACK_W13 = 0, MOE_PACK_W2 = 1, MOE_PACK_WS13 = 2, MOE_PACK_WS2 = 3,
  /* the transposed weights of the expert backward (moe_transpose_fp8_weights): each packed in tiles of
   * 256 rows like W2 */
  MOE_PACK_W13T = 4, MOE_PACK_W2T = 5, MOE_PACK_WS13T = 6, MOE_PACK_WS2T = 7
} moe_pack_which;

typedef struct {
  int32_t T;           /* tokens (>= 0; T == 0 is a no-op) */
  int32_t d_model;     /* d */
  int32_t n_routed;    /* E, 1..256 */
  int32_t n_shared;    /* Ks, >= 0 */
  int32_t top_k;       /* K, 1..min(E, 16) */
  int32_t inter_dim;   /* f, inner dim of one routed expert (and of one shared expert) */
  int32_t gate;        /* moe_gate */
  int32_t renorm;      /* 1: gates divided by their sum over the selected experts */
  int32_t act_dtype;   /* moe_dtype of u, h */
  int32_t w_dtype;     /* moe_dtype of expert weights */
  /* Group-limited routing (DeepSeek Technical Report: MoE Architecture, 2.3 device-limited routing,
   * M = 3 devices; 3.2 / 3.8 node-limited routing, M = 4 nodes). 0 / 0: no limit. Otherwise the E
   * experts form n_groups equal contiguous groups (1..16, dividing E); a group scores the largest
   * selection key among its experts; each token keeps the topk_groups best groups (ties to the lower
   * group index) and takes its top-K among their experts (K <= topk_groups * E / n_groups). Gates are
   * computed as without the limit. */
  int32_t n_groups;
  int32_t topk_groups;
} moe_config;

/* Layer weights (device pointers, read only).
 *  w13        [E, 2f, d]: rows 0..f-1 of each expert are W1 (gate), rows f..2f-1 are W3 (up).
 *  w2         [E, d, f]: W2 (down).
 *  w13_scale  [E, 2f/128, d/128] fp32, w2_scale [E, d/128, f/128] fp32: 128x128 block scales, fp8 only
 *             (NULL otherwise); a stored weight w is the E4M3 value q times its block's scale.
 *  ws13 [2fs, d], ws2 [d, fs] (+ ws13_scale [2fs/128, d/128], ws2_scale [d/128, fs/128]): the shared
 *             experts as one block; NULL when Ks == 0.
 *  w_gate     [E, d] fp32: the expert centroids e_i of the gate (logit z_{t,i} = u_t . e_i).
 *  logit_offset [E] fp32 or NULL: added to every logit before gating (a fixed per-expert skew).
 *  weight_layout  moe_weight_layout of w13, w2, ws13 and ws2 (all four alike; the scales keep their
 *             layout). MOE_LAYOUT_TILED holds the same values as the row layout, reordered by
 *             moe_pack_weights so that the expert GEMMs read every weight stage as one contiguous run;
 *             results are bit-identical. Zero (a zero-initialised struct) is the row layout. */
typedef struct {
  const void* w13;
  const void* w2;
  const float* w13_scale;
  const float* w2_scale;
  const void* ws13;
  const void* ws2;
  const float* ws13_scale;
  const float* ws2_scale;
  const float* w_gate;
  const float* logit_offset;
  int32_t weight_layout;
} moe_layer;

/* Bytes of workspace every call below needs for this configuration (host output). */
moe_status moe_workspace_size(const moe_config* cfg, size_t* bytes);

/* Router: logits, gating and top-K (DeepSeek Technical Report: MoE Architecture, 2.3 gate formula;
 * 3.3 and 5.3 [3]-[4] for sigmoid + bias).
 *  u        [T, d] act_dtype.
 *  bias     [E] fp32 selection bias, used only with MOE_GATE_SIGMOID_BIAS (NULL = zeros).
 *  topk_idx [T, K] int32 out: the selected routed experts of each token in ascending expert order.
 *           Keys are compared in fp32 and every token whose K-th and (K+1)-th keys are closer than
 *           delta_t = delta * max(1, |u_t| max_i |e_i| / sqrt(d)) is decided again from fp64 logits, so
 *           the set is the exact top-K; ties go to the lower expert index. delta (moe_route_margin) is
 *           2e-4 for softmax (logit units) and 4e-5 for sigmoid + bias (key units); the factor scales it
 *           with the size of the token's fp32 partial sums (|.| the Euclidean norm, e_i the rows of
 *           w_gate).
 *  topk_w   [T, K] fp32 out: gates, same order. Softmax: the probability over all E routed experts
 *           (renormalised over the K selected when cfg->renorm). Sigmoid: the affinity s, never s + b
 *           (renormalised when cfg->renorm). */
moe_status moe_route(const moe_config* cfg, const moe_layer* layer, const void* u, const float* bias,
                     int32_t* topk_idx, float* topk_w, void* ws, size_t ws_bytes, hipStream_t stream);

/* The base recheck margin delta of moe_route for this configuration's gating (host output). */
moe_status moe_route_margin(const moe_config* cfg, float* delta);

/* The router's fp32 logits alone (the first step of moe_route; for diagnostics and tests):
 * z [T, E] fp32 out, z[t][i] = u_t . e_i + logit_offset[i], computed exactly as moe_route computes the
 * keys it compares before the fp64 recheck (large bf16 batches: the centroids split into three bf16 parts
 * on the matrix cores, fp32 accumulation; otherwise fp64 vector FMAs, rounded to fp32 once). */
moe_status moe_router_logits(const moe_config* cfg, const moe_layer* layer, const void* u, float* z, void* ws,
                             size_t ws_bytes, hipStream_t stream);

/* Dispatch (DeepSeek Technical Report: MoE Architecture, 1.1: the routed sum of the layer runs over the
 * K experts of TopK(t) only, so each token's row goes to its K experts; 3.6 names this step, the
 * all-to-all dispatch of the multi-GPU design, whose payload is the E4M3 activation. On one GPU it is a
 * permutation: expert histogram, exclusive prefix sum and a stable order of the (token, slot) pairs by
 * expert. The 1x128 E4M3 quantization of u is not done here but by moe_expert_ffn, which gathers the
 * quantized rows of u through perm_src instead of reading a permuted copy).
 *  topk_idx [T, K] int32 in (as written by moe_route: distinct experts per token). A pair whose id is
 *           outside [0, E) or repeats an id of an earlier slot of the same token is dropped: it gets no
 *           row, is not counted, and its row_of entry is -1 (moe_combine adds nothing for it).
 *  counts   [E] int32 out: tokens per routed expert (sums to T*K when no pair is dropped).
 *  offsets  [E+1] int32 out: exclusive prefix sum of counts; rows of expert e are offsets[e]..offsets[e+1]-1.
 *  perm_src [T*K] int32 out: token of each row; tokens ascend within an expert. Entries past
 *           offsets[E] are not written.
 *  row_of   [T, K] int32 out: row of each (token, slot) pair, so perm_src[row_of[t][k]] == t, or -1. */
moe_status moe_dispatch(const moe_config* cfg, const int32_t* topk_idx, int32_t* counts, int32_t* offsets,
                        int32_t* perm_src, int32_t* row_of, void* ws, size_t ws_bytes, hipStream_t stream);

/* Expert FFNs as grouped GEMMs: for every routed expert e and its rows (from moe_dispatch), and for
 * the shared block over all T tokens, y = W2 (SiLU(W1 x) * (W3 x)).
 * fp8 weights: x is quantized per row per 128 columns, each 128-element partial product is scaled
 * and added into fp32 (DeepSeek Technical Report: MoE Architecture, 3.6), and SiLU(g) * v is
 * quantized again per 128 columns before W2.
 *  u         [T, d] act_dtype.   offsets [E+1], perm_src [T*K] from moe_dispatch.
 *  y_routed  [T*K, d] out (BF16 for E4M3 weights, else F32), rows in dispatch order.
 *  y_shared  [T, d] out, same dtype; NULL allowed only when Ks == 0. */
moe_status moe_expert_ffn(const moe_config* cfg, const moe_layer* layer, const void* u, const int32_t* offsets,
                          const int32_t* perm_src, void* y_routed, void* y_shared, void* ws, size_t ws_bytes,
                          hipStream_t stream);

/* Combine (DeepSeek Technical Report: MoE Architecture, 1.1 and 5.3 [1]: the layer output is the input
 * plus the shared experts' outputs plus the gate-weighted outputs of the selected routed experts; 3.6
 * sends the routed outputs back in BF16, the dtype of y_routed for E4M3 experts):
 *   h_t = u_t + y_shared_t + sum_k topk_w[t][k] * y_routed[row_of[t][k]],
 * summed in fp32 in that order (k ascending = expert ascending) and rounded once to act_dtype. A pair
 * with row_of[t][k] = -1 (dropped by moe_dispatch) adds nothing; any other entry must be a row below T*K.
 *  y_shared may be NULL when Ks == 0.  h [T, d] act_dtype out (must not alias the inputs). */
moe_status moe_combine(const moe_config* cfg, const void* u, const void* y_routed, const void* y_shared,
                       const int32_t* row_of, const float* topk_w, void* h, hipStream_t stream);

/* The whole layer (DeepSeek Technical Report: MoE Architecture, 1.1 "Shared Expert Isolation" formula
 * and 5.3 [1]; gating as in moe_route, experts as in moe_expert_ffn): moe_route, moe_dispatch,
 * moe_expert_ffn and moe_combine on `stream`, with every intermediate in the workspace. topk_idx [T, K]
 * and counts [E] are optional outputs (NULL to skip). The bias is read, never written: the update of
 * auxiliary-loss-free balancing is the separate call moe_update_bias, made after the step. */
moe_status moe_forward(const moe_config* cfg, const moe_layer* layer, const void* u, const float* bias, void* h,
                       int32_t* topk_idx, int32_t* counts, void* ws, size_t ws_bytes, hipStream_t stream);

/* Bytes of the static scratch that moe_forward_noalloc uses on each GPU (64 MiB: the V3-shaped layer up to
 * 256 tokens, a 2048-wide 64-expert layer up to 256 tokens). */
#define MOE_NOALLOC_SCRATCH_BYTES (64u << 20)

/* moe_forward without a caller workspace, for callers that cannot allocate device memory (code under HIP
 * graph capture, tight serving loops, harnesses that forbid hipMalloc). Same arguments, results and
 * errors as moe_forward; the intermediates live in a static array of MOE_NOALLOC_SCRATCH_BYTES bytes that
 * the library holds on every GPU it runs on until the process ends. The call allocates nothing (no
 * hipMalloc, hipFree or allocating library routine); the first call on a GPU looks up the address of that
 * GPU's array. A configuration whose moe_workspace_size exceeds MOE_NOALLOC_SCRATCH_BYTES returns
 * MOE_ERR_WORKSPACE before anything is launched. Every call on one GPU shares that GPU's array, so calls
 * that overlap on one GPU (other streams, other threads) race: serialize them. Nothing in the array
 * needs to start at any value; each call writes every intermediate before reading it. */
moe_status moe_forward_noalloc(const moe_config* cfg, const moe_layer* layer, const void* u, const float* bias, void* h,
                               int32_t* topk_idx, int32_t* counts, hipStream_t stream);

/* Bias update of auxiliary-loss-free balancing (DeepSeek Technical Report: MoE Architecture, 3.3):
 * b_i <- b_i - gamma if expert i is overloaded, b_i + gamma if underloaded, where overloaded means
 * counts[i] * E > T * K (load above the mean), underloaded the reverse; b_i is unchanged at the mean.
 * One fp32 subtraction per expert, in place.  counts [E] int32, bias [E] fp32 in/out. */
moe_status moe_update_bias(const moe_config* cfg, const int32_t* counts, float gamma, float* bias,
                           hipStream_t stream);

/* Input backward of the E4M3 experts (DeepSeek Technical Report: MoE Architecture, 3.6: the
 * activation backward GEMMs in FP8 with 1x128 activation tiles, 128x128 weight blocks and fp32
 * promotion every 128 elements). For every routed row r (dispatch order, as moe_expert_ffn's y_routed)
 * and every token of the shared block, given dy = dL/dy of the expert output, computes
 * dx = dL/dx of the expert input x (the token's u):
 *   g, v  = x [W1; W3]^T, recomputed in fp32 from x quantized 1x128 exactly as in the forward;
 *   da    = dy W2, with dy quantized 1x128 along d;
 *   dg    = da * v * sigmoid(g) * (1 + g (1 - sigmoid(g))),  dv = da * SiLU(g)   (fp32);
 *   dx    = [dg | dv] [W1; W3], with [dg | dv] quantized 1x128 along 2f.
 *  cfg      E4M3 experts (w_dtype MOE_FP8_E4M3), n_shared 0 or 1, inter_dim % 256 == 0 and
 *           2 * inter_dim <= 8192 (else MOE_ERR_UNSUPPORTED).
 *  layer    the forward weights (w13, w13_scale, ws13, ws13_scale are used), in either layout.
 *  layer_t  the same weights transposed (moe_transpose_fp8_weights, from the row layout): w13 =
 *           [W1; W3]^T [E, d, 2f] with scales [E, d/128, 2f/128], w2 = W2^T [E, f, d] with scales
 *           [E, f/128, d/128]; ws13 / ws2 likewise for the shared block. Either layout: MOE_LAYOUT_TILED
 *           with w13, w2, ws13, ws2 packed by MOE_PACK_W13T, MOE_PACK_W2T, MOE_PACK_WS13T, MOE_PACK_WS2T.
 *  u [T, d] bf16 (the layer input), offsets / perm_src as moe_dispatch returns them.
 *  dy_routed [T*K, d] bf16, dy_shared [T, d] bf16 (n_shared == 1); dx_routed [T*K, d] bf16 out,
 *  dx_shared [T, d] bf16 out.
 *  ws / ws_bytes: a workspace of at least moe_backward_workspace_size bytes (it covers the weight
 *  gradients of moe_expert_ffn_backward as well). */
moe_status moe_backward_workspace_size(const moe_config* cfg, size_t* bytes);
moe_status moe_expert_ffn_backward_input(const moe_config* cfg, const moe_layer* layer, const moe_layer* layer_t,
                                         const void* u, const int32_t* offsets, const int32_t* perm_src,
                                         const void* dy_routed, const void* dy_shared, void* dx_routed,
                                         void* dx_shared, void* ws, size_t ws_bytes, hipStream_t stream);

/* The full backward of the E4M3 experts: the input gradients above and/or the weight gradients
 * (DeepSeek Technical Report: MoE Architecture, 3.6: the weight backward GEMM in FP8 as well, weight
 * gradients kept in BF16). For every routed expert e over its rows (dispatch order) and for the shared
 * block over all T tokens:
 *   dW2      = dy^T a                [d, f]     a = SiLU(g) * v
 *   d[W1;W3] = [dg | dv]^T x         [2f, d]    (W1 rows first, the layout of w13)
 * with g, v, da, dg, dv as in moe_expert_ffn_backward_input. The contraction runs over the rows, so both
 * operands are quantized in 1x128 tiles along the rows, starting at the expert's first row (the last
 * tile padded with zero rows), promoted every 128 rows with the product of the two tiles' scales. The
 * cached activations enter as the values of their forward E4M3 copies: x quantized 1x128 along d, a
 * requantized 1x128 along f (as moe_expert_ffn does), each dequantized and requantized along the rows;
 * dy as given, [dg | dv] in fp32. An expert with no rows gets a zero gradient.
 *  dx_routed / dx_shared  as moe_expert_ffn_backward_input, or dx_routed = NULL to skip the input gradients.
 *  dw13 [E, 2f, d] bf16 and dw2 [E, d, f] bf16 out (the layouts of layer->w13 / w2), dws13 [2f, d] and
 *           dws2 [d, f] for the shared block (n_shared == 1), or dw13 = NULL to skip the weight gradients.
 *  At least one of dx_routed and dw13 is given (else MOE_ERR_INVALID_ARG). Outputs are overwritten, not
 *  accumulated. Other arguments, the workspace (moe_backward_workspace_size) and the limits as above. */
moe_status moe_expert_ffn_backward(const moe_config* cfg, const moe_layer* layer, const moe_layer* layer_t,
                                   const void* u, const int32_t* offsets, const int32_t* perm_src, const void* dy_routed,
                                   const void* dy_shared, void* dx_routed, void* dx_shared, void* dw13, void* dw2,
                                   void* dws13, void* dws2, void* ws, size_t ws_bytes, hipStream_t stream);

/* Expert weights in the row layout -> MOE_LAYOUT_TILED (a reordering of bytes: the expert GEMMs then read
 * each 128-byte K stage of a tile of 256 weight rows as 32 contiguous KB, in the order the matrix cores
 * take their operands; the values and every result are unchanged). For each expert (or the shared block)
 * and each tile n of 256 rows (W13: W1 rows 128 n .. 128 n + 127, then the W3 rows f + 128 n ..; W2: rows
 * 256 n ..) and K stage k (128 bytes of a row: 128 E4M3 or 64 bf16 values), 32 KB at offset
 * (n * stages + k) * 32768 of that expert's matrix: sixteen 2 KB blocks of 16 rows, and in block b the
 * 16-byte chunk c (0..7) of the block's row r (0..15) at byte 16 * (64 * (c / 4) + 16 * (c % 4) + r).
 * Scales are not touched.
 *  cfg    bf16 or fp8 weights (the sizes come from it; its T is not used).
 *  which  MOE_PACK_W13 (src/dst [E, 2f, d]), MOE_PACK_W2 ([E, d, f]), MOE_PACK_WS13 ([2 Ks f, d]),
 *         MOE_PACK_WS2 ([d, Ks f]); for the backward's transposed weights MOE_PACK_W13T ([E, d, 2f]),
 *         MOE_PACK_W2T ([E, f, d]), MOE_PACK_WS13T ([d, 2 Ks f]), MOE_PACK_WS2T ([Ks f, d]), all in tiles
 *         of 256 rows (f % 256 == 0 for W2T); the shared ones are a no-op when Ks == 0.
 *  src, dst  device buffers of the matrix's size, caller-owned, not overlapping (MOE_ERR_INVALID_ARG
 *         when src == dst).
 * Asynchronous on `stream`. */
moe_status moe_pack_weights(const moe_config* cfg, int32_t which, const void* src, void* dst, hipStream_t stream);

/* Transpose a batch of E4M3 matrices with their 128x128 block scales: qt[m] = q[m]^T ([cols, rows]),
 * scales_t[m] = scales[m]^T ([cols/128, rows/128]); the codes are unchanged, so a transposed block keeps
 * its scale. rows and cols are multiples of 128. Device pointers; qt must not alias q. */
moe_status moe_transpose_fp8_weights(const uint8_t* q, const float* scales, int32_t batch, int32_t rows, int32_t cols,
                                     uint8_t* qt, float* scales_t, hipStream_t stream);

/* Load-balance statistics of one routed batch (DeepSeek Technical Report: MoE Architecture, 1.2
 * expert-level balance loss L_ExpBal = alpha_1 * sum_i f_i * P_i, alpha_1 = 0.003 in 2.3; 3.3 the V3
 * sequence-wise balance loss, weight 0.0001, formula not printed). Readings: f_i = (tokens whose top-K
 * holds i) / T, with no E/K normalisation (sum_i f_i = K); P_i = mean over tokens of the probability of
 * expert i over all routed experts: softmax(z) in softmax mode, sigmoid(z) / sum_j sigmoid(z_j) in
 * sigmoid mode (the selection bias is not part of it); the sequence-wise loss is alpha_seq times the
 * mean over the T / seq_len sequences of sum_i f_i^b P_i^b taken within each sequence.
 *  z        [T, E] fp32: router logits, as moe_router_logits returns them.
 *  topk_idx [T, K] int32: the selection, as moe_route returns it.
 *  seq_len  tokens per sequence (consecutive tokens): T itself, or a multiple of 64 that divides T
 *           (otherwise MOE_ERR_INVALID_ARG if it does not divide T, MOE_ERR_UNSUPPORTED if it is not a
 *           multiple of 64).
 *  f, P     [E] fp32 out; loss [2] fp32 out: loss[0] = alpha_expert * sum f P, loss[1] = the
 *           sequence-wise loss. All sums run in fp64 in a fixed order (the result is deterministic).
 *  ws / ws_bytes: the layer workspace (moe_workspace_size); device pointers throughout. */
moe_status moe_balance_stats(const moe_config* cfg, const float* z, const int32_t* topk_idx, int32_t seq_len,
                             float alpha_expert, float alpha_seq, float* f, float* P, float* loss, void* ws,
                             size_t ws_bytes, hipStream_t stream);

/* Offline weight preparation (DeepSeek Technical Report: MoE Architecture, 3.6, 128x128 weight blocks):
 * quantizes `batch` fp32 matrices w [batch, rows, cols] (rows, cols multiples of 128) to E4M3 codes
 * q [batch, rows, cols] uint8 and block scales [batch, rows/128, cols/128] fp32 with
 * s = amax/448, q = E4M3(w * (448/amax)) (nearest-even, saturating; s = 1 for an all-zero block). */
moe_status moe_quantize_weights(const float* w, int32_t batch, int32_t rows, int32_t cols, uint8_t* q,
                                float* scales, hipStream_t stream);

/* Activation quantization, 1x128 tiles (same report, 3.6): x [rows, cols] of dtype x_dtype
 * (F32 or BF16; cols % 128 == 0) -> q [rows, cols] E4M3 codes and scales [rows, cols/128] fp32, with the
 * same scale rule as moe_quantize_weights. */
moe_status moe_quantize_act(const void* x, int32_t x_dtype, int32_t rows, int32_t cols, uint8_t* q,
                            float* scales, hipStream_t stream);

/* Stage marks for timing (a measurement aid, not part of the layer). After moe_set_timing_events(ev, n)
 * with n >= MOE_NUM_MARKS, calls made on this thread record ev[m] on their stream at each mark m they pass:
 * moe_forward records all of them; moe_route marks ROUTE_BEGIN..ROUTE_END, moe_dispatch DISPATCH_END,
 * moe_expert_ffn QUANT_END..DOWN_END, moe_combine COMBINE_END. The events are created and owned by the
 * caller (host handles); ev = NULL switches the marks off. Returns MOE_ERR_INVALID_ARG for 0 < n < NUM_MARKS. */
typedef enum {
  MOE_MARK_ROUTE_BEGIN = 0,  /* before the router kernels */
  MOE_MARK_ROUTE_END,        /* after the router (topk_idx, topk_w ready) */
  MOE_MARK_DISPATCH_END,     /* after histogram, scan and permutation */
  MOE_MARK_QUANT_END,        /* after the tile schedule and (E4M3) the 1x128 activation quantization */
  MOE_MARK_GATEUP_END,       /* after the gate/up + SwiGLU grouped GEMM */
  MOE_MARK_DOWN_END,         /* after the down grouped GEMM */
  MOE_MARK_COMBINE_END,      /* after the combine */
  MOE_NUM_MARKS
} moe_mark;
moe_status moe_set_timing_events(hipEvent_t* events, int32_t n);

/* Message for the last non-OK status returned on this thread ("" if none). Host string, owned by the
 * library, valid until the next call on this thread. */
const char* moe_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* MOE_MI355X_H */
