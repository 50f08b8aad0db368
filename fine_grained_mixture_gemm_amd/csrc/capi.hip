// C ABI of libmoe: argument validation, workspace layout and the launch sequence of each entry point.
// Every call validates synchronously, then enqueues kernels on the caller's stream; nothing is allocated.
#include <algorithm>
#include <cstdarg>
#include <cstdio>
#include <initializer_list>
#include <mutex>
#include <string>
#include <utility>

#include "common.h"
#include "kernels.h"

using namespace moe;

namespace {

thread_local std::string g_err;
thread_local hipEvent_t g_marks[MOE_NUM_MARKS];
thread_local bool g_marks_on = false;

void mark(int m, hipStream_t s) {
  if (g_marks_on) (void)hipEventRecord(g_marks[m], s);
}

moe_status fail(moe_status s, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_err = buf;
  return s;
}

moe_status hip_status(hipError_t e, const char* what) {
  if (e == hipSuccess) return MOE_OK;
  return fail(MOE_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

#define MOE_TRY(x)                      \
  do {                                  \
    moe_status _s = (x);                \
    if (_s != MOE_OK) return _s;        \
  } while (0)

// Tokens whose K-th and (K+1)-th fp32 keys differ by less than this (times max(1, |u_t| max_i |e_i| /
// sqrt(d)), the size of the token's partial sums against token rows of RMS 1 and centroids of norm 1) are
// decided from fp64 logits. The base margins are at least 20x the largest fp32 key error measured
// against fp64 logits on the synthetic layers: 1.7e-6 for sigmoid keys at d = 7168, 6.4e-6 for softmax
// keys (logits) at d = 1024.
constexpr float kRecheckDeltaSigmoid = 4e-5f;
constexpr float kRecheckDeltaSoftmax = 2e-4f;

bool use_mfma_gemm(const moe_config* c) { return c->w_dtype != MOE_F32; }
// bf16 tokens take the MFMA logits from T * E >= 2^16 (256 tokens of 256 experts, or the 2B layer's 2048
// tokens of 63 experts); below that the vector-ALU logits split over d are faster (a decode step). Route
// stage against a 2^17 threshold: 2B layer 0.060 -> 0.051 ms, V3 layer at 256 / 384 tokens 0.089 / 0.114 ->
// 0.082 / 0.082 ms.
constexpr long long kMfmaRouterMin = 1LL << 16;
bool use_mfma_router(const moe_config* c) {
  return c->act_dtype == MOE_BF16 && c->d_model % 64 == 0 && (long long)c->T * c->n_routed >= kMfmaRouterMin;
}

// expert outputs: bf16 for E4M3 experts (the combine payload), fp32 otherwise
int esz_y(const moe_config* c) { return c->w_dtype == MOE_FP8_E4M3 ? 2 : 4; }

moe_status check_cfg(const moe_config* c) {
  if (!c) return fail(MOE_ERR_INVALID_ARG, "cfg is NULL");
  if (c->T < 0 || c->d_model <= 0 || c->n_routed <= 0 || c->n_shared < 0 || c->top_k <= 0 || c->inter_dim <= 0)
    return fail(MOE_ERR_INVALID_ARG, "sizes must be positive (T >= 0): T=%d d=%d E=%d Ks=%d K=%d f=%d", c->T,
                c->d_model, c->n_routed, c->n_shared, c->top_k, c->inter_dim);
  if (c->top_k > c->n_routed) return fail(MOE_ERR_INVALID_ARG, "top_k=%d exceeds n_routed=%d", c->top_k, c->n_routed);
  if (c->gate != MOE_GATE_SOFTMAX && c->gate != MOE_GATE_SIGMOID_BIAS) return fail(MOE_ERR_INVALID_ARG, "bad gate %d", c->gate);
  if (c->renorm != 0 && c->renorm != 1) return fail(MOE_ERR_INVALID_ARG, "renorm must be 0 or 1");
  if (c->act_dtype != MOE_F32 && c->act_dtype != MOE_BF16) return fail(MOE_ERR_INVALID_ARG, "bad act_dtype %d", c->act_dtype);
  if (c->w_dtype != MOE_F32 && c->w_dtype != MOE_BF16 && c->w_dtype != MOE_FP8_E4M3)
    return fail(MOE_ERR_INVALID_ARG, "bad w_dtype %d", c->w_dtype);
  if (c->n_routed > 256) return fail(MOE_ERR_UNSUPPORTED, "n_routed=%d > 256 (one wave holds at most 256 keys)", c->n_routed);
  if (c->n_groups != 0 || c->topk_groups != 0) {
    if (c->n_groups < 1 || c->n_routed % c->n_groups || c->topk_groups < 1 || c->topk_groups > c->n_groups ||
        c->top_k > c->topk_groups * (c->n_routed / c->n_groups))
      return fail(MOE_ERR_INVALID_ARG, "bad group limit: n_groups=%d topk_groups=%d (E=%d K=%d)", c->n_groups,
                  c->topk_groups, c->n_routed, c->top_k);
    if (c->n_groups > 16) return fail(MOE_ERR_UNSUPPORTED, "n_groups=%d > 16", c->n_groups);
  }
  if (c->top_k > 16) return fail(MOE_ERR_UNSUPPORTED, "top_k=%d > 16", c->top_k);
  if (c->d_model > 8192) return fail(MOE_ERR_UNSUPPORTED, "d_model=%d > 8192 (fp64 router recheck)", c->d_model);
  const bool pair_ok = (c->act_dtype == MOE_F32 && c->w_dtype == MOE_F32) ||
                       (c->act_dtype == MOE_BF16 && (c->w_dtype == MOE_BF16 || c->w_dtype == MOE_FP8_E4M3));
  if (!pair_ok) return fail(MOE_ERR_UNSUPPORTED, "unsupported (act, weight) dtype pair (%d, %d)", c->act_dtype, c->w_dtype);
  if (c->w_dtype != MOE_F32 && (c->d_model % 256 != 0 || c->inter_dim % 128 != 0))
    return fail(MOE_ERR_UNSUPPORTED, "bf16/fp8 experts need d %% 256 == 0 and f %% 128 == 0 (d=%d f=%d)", c->d_model,
                c->inter_dim);
  // the E4M3 GEMM holds one weight block scale per 128-element K block in one lane of a wave
  if (c->w_dtype == MOE_FP8_E4M3 && (long long)std::max(1, c->n_shared) * c->inter_dim > 8192)
    return fail(MOE_ERR_UNSUPPORTED, "E4M3 experts need max(1, n_shared) * inter_dim <= 8192 (got %d * %d)",
                c->n_shared, c->inter_dim);
  const long long rows = (long long)c->T * c->top_k;
  if (rows >= (1LL << 31) || (long long)c->n_shared * c->inter_dim >= (1LL << 30))
    return fail(MOE_ERR_UNSUPPORTED, "T*K or Ks*f too large");
  // the matrix-core kernels address activations and one expert's weights with 32-bit byte offsets
  const long long fs = (long long)c->n_shared * c->inter_dim;
  const long long big = std::max({(long long)c->T * c->d_model * 2, rows * c->inter_dim * 2, (long long)c->T * fs * 2,
                                  2LL * std::max((long long)c->inter_dim, fs) * c->d_model * 2});
  if (c->w_dtype != MOE_F32 && big >= (1LL << 32))
    return fail(MOE_ERR_UNSUPPORTED, "an activation or expert weight array exceeds 4 GiB");
  return MOE_OK;
}

struct Layout {
  size_t z, z64, wg_split, zpart, recheck_count, recheck_list, wn2, un2;
  size_t chunk_counts, mt_prefix, xsched;
  size_t uq, us, xsb_r, xsb_s, a_r, a_s, as_r, as_s;
  size_t f_idx, f_w, f_counts, f_offsets, f_perm, f_rowof, f_yr, f_ys;
  size_t bal_psum, bal_cnt, bal_seqp, bal_seqn, bal_seq;
  size_t total;
};

Layout layout(const moe_config* c) {
  Layout L{};
  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t at = off;
    off = align_up(off + bytes, 256);
    return at;
  };
  const size_t T = c->T, E = c->n_routed, K = c->top_k, d = c->d_model, f = c->inter_dim;
  const size_t fs = (size_t)c->n_shared * f;
  const size_t rows = T * K;
  const bool fp8 = c->w_dtype == MOE_FP8_E4M3;
  const size_t esz_a = c->w_dtype == MOE_F32 ? 4 : (c->w_dtype == MOE_BF16 ? 2 : 1);
  L.z = take(T * E * 4);
  L.z64 = take(T * E * (use_mfma_router(c) ? 16 : 8));   // MFMA logits: also up to four fp32 partial slices
  L.wg_split = take(use_mfma_router(c) ? 3 * E * d * 2 : 0);
  int klen = 0;
  const int ksplit = use_mfma_router(c) ? 1 : router_ksplit((int)T, (int)E, (int)d, klen);
  L.zpart = take(ksplit > 1 ? (size_t)ksplit * T * E * 8 : 0);
  L.recheck_count = take(16);
  L.recheck_list = take(T * 4);
  L.wn2 = take(E * 4);
  L.un2 = take((use_mfma_router(c) ? 4 : (size_t)ksplit) * T * 4);   // token norms per slice of d
  const size_t nch = dispatch_chunks(c->T);
  L.chunk_counts = take(nch * E * 4);
  L.mt_prefix = take((E + 1) * 4);
  L.xsched = take(2 * (kSchedRange + kSchedCount) * 4);
  L.uq = take(fp8 ? T * d : 0);
  L.us = take(fp8 ? T * (d / 128) * 4 : 0);
  // the same scales block-major in the dispatched order (routed rows) and in token order (shared experts),
  // read by the matrix-core gate/up GEMM
  const bool xsb = fp8 && use_mfma_gemm(c) && c->T > gemm_decode_max_tokens();
  L.xsb_r = take(xsb ? rows * (d / 128) * 4 : 0);
  L.xsb_s = take(xsb && fs > 0 ? T * (d / 128) * 4 : 0);
  L.a_r = take(rows * f * esz_a);
  L.a_s = take(T * fs * esz_a);
  L.as_r = take(fp8 ? rows * (f / 128) * 4 : 0);
  L.as_s = take(fp8 ? T * (fs / 128) * 4 : 0);
  L.f_idx = take(rows * 4);
  L.f_w = take(rows * 4);
  L.f_counts = take(E * 4);
  L.f_offsets = take((E + 1) * 4);
  L.f_perm = take(rows * 4);
  L.f_rowof = take(rows * 4);
  L.f_yr = take(rows * d * esz_y(c));
  L.f_ys = take(T * d * esz_y(c));
  const size_t bch = balance_chunks_for(c->T);
  L.bal_psum = take(bch * E * 8);
  L.bal_cnt = take(bch * E * 4);
  const size_t bsq = balance_sequences_max(c->T);
  L.bal_seqp = take(bsq * E * 8);
  L.bal_seqn = take(bsq * E * 4);
  L.bal_seq = take(bsq * 8);
  L.total = off + 256;   // room to align the caller's base pointer up to 256 bytes
  return L;
}

moe_status check_ws(const moe_config* c, void* ws, size_t ws_bytes, uint8_t** base, Layout* L) {
  *L = layout(c);
  if (!ws) return fail(MOE_ERR_WORKSPACE, "workspace is NULL");
  if (ws_bytes < L->total) return fail(MOE_ERR_WORKSPACE, "workspace %zu bytes < required %zu", ws_bytes, L->total);
  *base = reinterpret_cast<uint8_t*>(align_up(reinterpret_cast<uintptr_t>(ws), 256));
  return MOE_OK;
}

int device_cus() {
  static thread_local int cached_dev = -1, cached_cus = 0;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 256;
  if (dev != cached_dev) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
    cached_dev = dev;
    cached_cus = n;
  }
  return cached_cus;
}

// Workspace of the E4M3 input backward of the experts (its own size query).
struct BwdLayout {
  size_t uq, us, mt_prefix, xsched_a, xsched_b;
  size_t dyq_r, dys_r, dyq_s, dys_s, da_r, da_s, gv_r, gv_s, dgq_r, dgs_r, dgq_s, dgs_s;
  // weight gradients: row-block prefix, operands quantized along the rows (codes [C][rpad], scales
  // [row block][C])
  size_t pblk, wq_dy, ws_dy, wq_a, ws_a, wq_dgv, ws_dgv, wq_x, ws_x;
  int nblk;
  size_t rpad;
  size_t total;
};

BwdLayout bwd_layout(const moe_config* c) {
  BwdLayout L{};
  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t at = off;
    off = align_up(off + bytes, 256);
    return at;
  };
  const size_t T = c->T, E = c->n_routed, d = c->d_model, f = c->inter_dim, fs = (size_t)c->n_shared * f;
  const size_t rows = T * c->top_k;
  L.uq = take(T * d);
  L.us = take(T * (d / 128) * 4);
  L.mt_prefix = take((E + 1) * 4);
  L.xsched_a = take(2 * (kSchedRange + kSchedCount) * 4);
  L.xsched_b = take(2 * (kSchedRange + kSchedCount) * 4);
  L.dyq_r = take(rows * d);
  L.dys_r = take(rows * (d / 128) * 4);
  L.dyq_s = take(T * d * (fs > 0));
  L.dys_s = take(T * (d / 128) * 4 * (fs > 0));
  L.da_r = take(rows * f * 4);
  L.da_s = take(T * fs * 4);
  L.gv_r = take(rows * 2 * f * 4);
  L.gv_s = take(T * 2 * fs * 4);
  L.dgq_r = take(rows * 2 * f);
  L.dgs_r = take(rows * (2 * f / 128) * 4);
  L.dgq_s = take(T * 2 * fs);
  L.dgs_s = take(T * (2 * fs / 128) * 4);
  L.nblk = wgrad_row_blocks_max(c->T, c->top_k, c->n_routed, fs > 0);
  L.rpad = (size_t)L.nblk * 128;
  const size_t nb = L.nblk;
  L.pblk = take((E + 2 + 18) * 4);
  L.wq_dy = take(d * L.rpad);
  L.ws_dy = take(nb * d * 4);
  L.wq_a = take(f * L.rpad);
  L.ws_a = take(nb * f * 4);
  L.wq_dgv = take(2 * f * L.rpad);
  L.ws_dgv = take(nb * 2 * f * 4);
  L.wq_x = take(d * L.rpad);
  L.ws_x = take(nb * d * 4);
  L.total = off + 256;
  return L;
}

moe_status check_bwd_cfg(const moe_config* c) {
  MOE_TRY(check_cfg(c));
  if (c->w_dtype != MOE_FP8_E4M3) return fail(MOE_ERR_UNSUPPORTED, "the expert input backward is built for E4M3 experts");
  if (c->n_shared > 1) return fail(MOE_ERR_UNSUPPORTED, "the expert input backward takes at most one shared expert");
  if (c->inter_dim % 256) return fail(MOE_ERR_UNSUPPORTED, "the expert input backward needs inter_dim %% 256 == 0");
  if (2 * c->inter_dim > 8192) return fail(MOE_ERR_UNSUPPORTED, "the expert input backward needs 2 * inter_dim <= 8192");
  return MOE_OK;
}

// Weight gradients (after the g/v and da GEMMs of the backward have filled gv and da): the row-block
// prefix, the four operands quantized along the rows, then dW2 = dy^T a and d[W1; W3] = [dg | dv]^T x.
moe_status weight_gradients(const moe_config* c, const BwdLayout& L, uint8_t* base, const void* u,
                            const int32_t* offsets, const int32_t* perm, const void* dy_r, const void* dy_s,
                            void* dw13, void* dw2, void* dws13, void* dws2, hipStream_t s) {
  const bool sh = c->n_shared > 0;
  const int E = c->n_routed, d = c->d_model, f = c->inter_dim;
  int32_t* pblk = reinterpret_cast<int32_t*>(base + L.pblk);
  auto F = [&](size_t o) { return reinterpret_cast<float*>(base + o); };
  MOE_TRY(hip_status(launch_wgrad_prefix(offsets, E, c->T, sh, pblk, s), "row-block prefix launch"));
  WgQuantArgs q{};
  q.offsets = offsets;
  q.perm = perm;
  q.pblk = pblk;
  q.E = E;
  q.T = c->T;
  q.fg = f;
  q.rpad = L.rpad;
  q.gv_r = F(L.gv_r);
  q.gv_s = F(L.gv_s);
  q.da_r = F(L.da_r);
  q.da_s = F(L.da_s);
  auto quant = [&](int src, int C, const void* br, const void* bs, size_t wq, size_t wsc) {
    q.C = C;
    q.bf_r = static_cast<const uint16_t*>(br);
    q.bf_s = static_cast<const uint16_t*>(bs);
    q.qt = base + wq;
    q.st = F(wsc);
    return hip_status(launch_wgrad_quant(q, src, L.nblk, s), "row quantization launch");
  };
  MOE_TRY(quant(kWgSrcDy, d, dy_r, dy_s, L.wq_dy, L.ws_dy));
  MOE_TRY(quant(kWgSrcA, f, nullptr, nullptr, L.wq_a, L.ws_a));
  MOE_TRY(quant(kWgSrcDgv, 2 * f, nullptr, nullptr, L.wq_dgv, L.ws_dgv));
  MOE_TRY(quant(kWgSrcX, d, u, u, L.wq_x, L.ws_x));
  WgGemmArgs g{};
  g.pblk = pblk;
  g.E = E;
  g.shared = sh ? 1 : 0;
  g.rpad = L.rpad;
  // dW2 [d][f]: rows from dy, columns from a
  g.M = d;
  g.N = f;
  g.A = base + L.wq_a;
  g.As = F(L.ws_a);
  g.B = base + L.wq_dy;
  g.Bs = F(L.ws_dy);
  g.out_r = static_cast<uint16_t*>(dw2);
  g.out_s = static_cast<uint16_t*>(dws2);
  g.xcount = pblk + E + 2;
  const int grid = std::max(8, device_cus());
  MOE_TRY(hip_status(launch_wgrad_gemm(g, grid, s), "dW2 GEMM launch"));
  // d[W1; W3] [2f][d]: rows from [dg | dv], columns from x
  g.M = 2 * f;
  g.N = d;
  g.A = base + L.wq_x;
  g.As = F(L.ws_x);
  g.B = base + L.wq_dgv;
  g.Bs = F(L.ws_dgv);
  g.out_r = static_cast<uint16_t*>(dw13);
  g.out_s = static_cast<uint16_t*>(dws13);
  g.xcount = pblk + E + 11;
  MOE_TRY(hip_status(launch_wgrad_gemm(g, grid, s), "dW13 GEMM launch"));
  return MOE_OK;
}

// The kernels read and write activations, expert weights and expert outputs in 16-byte pieces: each
// such buffer (when given) must start on a 16-byte boundary.
moe_status check_aligned16(std::initializer_list<std::pair<const char*, const void*>> bufs) {
  for (const auto& b : bufs)
    if (b.second && (reinterpret_cast<uintptr_t>(b.second) & 15))
      return fail(MOE_ERR_INVALID_ARG, "%s is not 16-byte aligned", b.first);
  return MOE_OK;
}

moe_status check_layer_router(const moe_layer* l) {
  if (!l) return fail(MOE_ERR_INVALID_ARG, "layer is NULL");
  if (!l->w_gate) return fail(MOE_ERR_INVALID_ARG, "layer->w_gate is NULL");
  return check_aligned16({{"layer->w_gate", l->w_gate}});
}

moe_status check_layer_experts(const moe_config* c, const moe_layer* l) {
  if (!l) return fail(MOE_ERR_INVALID_ARG, "layer is NULL");
  if (!l->w13 || !l->w2) return fail(MOE_ERR_INVALID_ARG, "layer->w13 / w2 is NULL");
  if (l->weight_layout != MOE_LAYOUT_ROWS && l->weight_layout != MOE_LAYOUT_TILED)
    return fail(MOE_ERR_INVALID_ARG, "bad weight_layout %d", l->weight_layout);
  if (l->weight_layout == MOE_LAYOUT_TILED && c->w_dtype == MOE_F32)
    return fail(MOE_ERR_UNSUPPORTED, "the tiled weight layout is for bf16 and fp8 weights");
  const bool fp8 = c->w_dtype == MOE_FP8_E4M3;
  if (fp8 && (!l->w13_scale || !l->w2_scale)) return fail(MOE_ERR_INVALID_ARG, "fp8 weights need w13_scale and w2_scale");
  if (c->n_shared > 0) {
    if (!l->ws13 || !l->ws2) return fail(MOE_ERR_INVALID_ARG, "n_shared > 0 needs ws13 and ws2");
    if (fp8 && (!l->ws13_scale || !l->ws2_scale)) return fail(MOE_ERR_INVALID_ARG, "fp8 shared weights need scales");
  }
  return check_aligned16({{"layer->w13", l->w13}, {"layer->w2", l->w2}, {"layer->ws13", l->ws13}, {"layer->ws2", l->ws2}});
}

RouteArgs route_args(const moe_config* c, const moe_layer* l, const void* u, const float* bias, int32_t* idx, float* w,
                     uint8_t* base, const Layout& L) {
  RouteArgs a{};
  a.u = u;
  a.u_bf16 = c->act_dtype == MOE_BF16;
  a.use_mfma = use_mfma_router(c);
  a.wg = l->w_gate;
  a.off = l->logit_offset;
  a.bias = c->gate == MOE_GATE_SIGMOID_BIAS ? bias : nullptr;
  a.T = c->T;
  a.E = c->n_routed;
  a.d = c->d_model;
  a.K = c->top_k;
  a.gate = c->gate;
  a.renorm = c->renorm;
  a.n_groups = c->n_groups;
  a.topk_groups = c->topk_groups;
  a.delta = c->gate == MOE_GATE_SOFTMAX ? kRecheckDeltaSoftmax : kRecheckDeltaSigmoid;
  a.wn2 = reinterpret_cast<float*>(base + L.wn2);
  a.un2 = reinterpret_cast<float*>(base + L.un2);
  a.z = reinterpret_cast<float*>(base + L.z);
  a.z64 = reinterpret_cast<double*>(base + L.z64);
  a.wg_split = reinterpret_cast<uint16_t*>(base + L.wg_split);
  a.ksplit = a.use_mfma ? 1 : router_ksplit(a.T, a.E, a.d, a.klen);
  a.zpart = reinterpret_cast<double*>(base + L.zpart);
  a.recheck_count = reinterpret_cast<int*>(base + L.recheck_count);
  a.recheck_list = reinterpret_cast<int*>(base + L.recheck_list);
  a.topk_idx = idx;
  a.topk_w = w;
  return a;
}

moe_status do_route(const moe_config* c, const moe_layer* l, const void* u, const float* bias, int32_t* idx, float* w,
                    uint8_t* base, const Layout& L, hipStream_t s) {
  const RouteArgs a = route_args(c, l, u, bias, idx, w, base, L);
  mark(MOE_MARK_ROUTE_BEGIN, s);
  MOE_TRY(hip_status(launch_route(a, s), "router launch"));
  mark(MOE_MARK_ROUTE_END, s);
  return MOE_OK;
}

moe_status do_dispatch(const moe_config* c, const int32_t* idx, int32_t* counts, int32_t* offsets, int32_t* perm,
                       int32_t* row_of, uint8_t* base, const Layout& L, hipStream_t s) {
  DispatchArgs a{};
  a.topk_idx = idx;
  a.T = c->T;
  a.E = c->n_routed;
  a.K = c->top_k;
  a.chunk_counts = reinterpret_cast<int32_t*>(base + L.chunk_counts);
  a.counts = counts;
  a.offsets = offsets;
  a.perm_src = perm;
  a.row_of = row_of;
  MOE_TRY(hip_status(launch_dispatch(a, s), "dispatch launch"));
  mark(MOE_MARK_DISPATCH_END, s);
  return MOE_OK;
}

moe_status do_ffn(const moe_config* c, const moe_layer* l, const void* u, const int32_t* offsets, const int32_t* perm,
                  void* y_r, void* y_s, uint8_t* base, const Layout& L, hipStream_t s) {
  if (c->T == 0) return MOE_OK;
  const bool fp8 = c->w_dtype == MOE_FP8_E4M3;
  const bool mfma = use_mfma_gemm(c);
  const int bm = mfma ? gemm_mfma_bm() : gemm_simt_bm();
  int32_t* mt_prefix = reinterpret_cast<int32_t*>(base + L.mt_prefix);
  int32_t* xrange = reinterpret_cast<int32_t*>(base + L.xsched);
  int32_t* xcount = xrange + 2 * kSchedRange;
  const int fs = c->n_shared * c->inter_dim;
  // a decode-sized E4M3 batch streams the touched experts' weights with its own kernels (no tile list)
  const bool decode = fp8 && c->T <= gemm_decode_max_tokens();
  // E4M3 on the matrix-core tiles: the schedule is computed by the activation quantization's launch
  const bool fused = fp8 && mfma && !decode;
  SchedArgs sa{offsets, c->n_routed, c->T, bm, {c->inter_dim / 128, c->d_model / 256},
               {fs / 128, fs > 0 ? c->d_model / 256 : 0}, mt_prefix, xrange, xcount};
  if (mfma && !decode && !fused) {
    MOE_TRY(hip_status(launch_schedule_mfma(offsets, c->n_routed, c->T, bm, sa.nt_r, sa.nt_s, mt_prefix, xrange, xcount, s),
                       "schedule launch"));
  } else if (!mfma) {
    MOE_TRY(hip_status(launch_schedule(offsets, c->n_routed, bm, mt_prefix, s), "schedule launch"));
  }
  GemmArgs g{};
  g.E = c->n_routed;
  g.T = c->T;
  g.d = c->d_model;
  g.f = c->inter_dim;
  g.fs = fs;
  g.offsets = offsets;
  g.perm_src = perm;
  g.mt_prefix = mt_prefix;
  g.xrange = xrange;
  g.xcount = xcount;
  g.packed = l->weight_layout == MOE_LAYOUT_TILED;
  const uint8_t* xin = static_cast<const uint8_t*>(u);
  const float* xs = nullptr;
  if (fused) {
    MOE_TRY(hip_status(launch_quant_act_schedule(u, c->T, c->d_model, base + L.uq, reinterpret_cast<float*>(base + L.us), sa, s),
                       "activation quantization and schedule launch"));
    xin = base + L.uq;
    xs = reinterpret_cast<const float*>(base + L.us);
  } else if (fp8) {
    MOE_TRY(hip_status(launch_quant_act(u, true, c->T, c->d_model, base + L.uq, reinterpret_cast<float*>(base + L.us), s),
                       "activation quantization launch"));
    xin = base + L.uq;
    xs = reinterpret_cast<const float*>(base + L.us);
  }
  // matrix-core E4M3 path: token scales and the scales of a block-major (one stage's scales of a tile are
  // contiguous)
  const bool xsb = fp8 && mfma && !decode;
  const long long rows = (long long)c->T * c->top_k;
  if (xsb) {
    const int kblk = c->d_model / 128;
    MOE_TRY(hip_status(launch_scales_by_block(xs, kblk, perm, offsets + c->n_routed, (int)rows,
                                              reinterpret_cast<float*>(base + L.xsb_r), (int)rows, fs > 0 ? c->T : 0,
                                              reinterpret_cast<float*>(base + L.xsb_s), c->T, s),
                       "scale layout launch"));
  }
  mark(MOE_MARK_QUANT_END, s);
  // gate/up + SwiGLU
  g.w_routed = static_cast<const uint8_t*>(l->w13);
  g.w_shared = static_cast<const uint8_t*>(l->ws13);
  g.ws_routed = l->w13_scale;
  g.ws_shared = l->ws13_scale;
  g.x_routed = xin;
  g.x_shared = xin;
  g.xs_routed = xsb ? reinterpret_cast<const float*>(base + L.xsb_r) : xs;
  g.xs_shared = xsb ? reinterpret_cast<const float*>(base + L.xsb_s) : xs;
  g.xs_ld_routed = g.os_ld_routed = xsb ? (int)rows : 0;
  g.xs_ld_shared = g.os_ld_shared = xsb ? c->T : 0;
  g.out_routed = base + L.a_r;
  g.out_shared = base + L.a_s;
  g.out_scale_routed = reinterpret_cast<float*>(base + L.as_r);
  g.out_scale_shared = reinterpret_cast<float*>(base + L.as_s);
  if (decode) {
    MOE_TRY(hip_status(launch_gemm_decode(g, true, s), "gate/up GEMM launch"));
  } else if (mfma) {
    const int grid = device_cus() / 8 * 8;
    MOE_TRY(hip_status(launch_gemm_mfma(g, fp8, true, grid, s), "gate/up GEMM launch"));
  } else {
    const int mt_bound = (int)((rows + bm - 1) / bm) + c->n_routed;
    const int mt_s = fs > 0 ? cdiv(c->T, bm) : 0;
    const int tiles = mt_bound * cdiv(c->inter_dim, 32) + mt_s * cdiv(fs, 32);
    MOE_TRY(hip_status(launch_gemm_simt(g, true, tiles, s), "gate/up GEMM launch"));
  }
  mark(MOE_MARK_GATEUP_END, s);
  // down
  g.w_routed = static_cast<const uint8_t*>(l->w2);
  g.w_shared = static_cast<const uint8_t*>(l->ws2);
  g.ws_routed = l->w2_scale;
  g.ws_shared = l->ws2_scale;
  g.x_routed = base + L.a_r;
  g.x_shared = base + L.a_s;
  g.xs_routed = reinterpret_cast<const float*>(base + L.as_r);
  g.xs_shared = reinterpret_cast<const float*>(base + L.as_s);
  g.out_routed = static_cast<uint8_t*>(y_r);
  g.out_shared = static_cast<uint8_t*>(y_s);
  g.out_scale_routed = nullptr;
  g.out_scale_shared = nullptr;
  g.xrange = xrange + kSchedRange;
  g.xcount = xcount + kSchedCount;
  if (decode) {
    MOE_TRY(hip_status(launch_gemm_decode(g, false, s), "down GEMM launch"));
  } else if (mfma) {
    const int grid = device_cus() / 8 * 8;
    MOE_TRY(hip_status(launch_gemm_mfma(g, fp8, false, grid, s), "down GEMM launch"));
  } else {
    const int mt_bound = (int)((rows + bm - 1) / bm) + c->n_routed;
    const int mt_s = fs > 0 ? cdiv(c->T, bm) : 0;
    const int nt = cdiv(c->d_model, 64);
    MOE_TRY(hip_status(launch_gemm_simt(g, false, mt_bound * nt + mt_s * nt, s), "down GEMM launch"));
  }
  mark(MOE_MARK_DOWN_END, s);
  return MOE_OK;
}

}  // namespace

extern "C" {

const char* moe_last_error(void) { return g_err.c_str(); }

moe_status moe_set_timing_events(hipEvent_t* events, int32_t n) {
  if (!events || n == 0) {
    g_marks_on = false;
    return MOE_OK;
  }
  if (n < MOE_NUM_MARKS) return fail(MOE_ERR_INVALID_ARG, "need %d events, got %d", (int)MOE_NUM_MARKS, n);
  for (int i = 0; i < MOE_NUM_MARKS; ++i) g_marks[i] = events[i];
  g_marks_on = true;
  return MOE_OK;
}

moe_status moe_route_margin(const moe_config* cfg, float* delta) {
  MOE_TRY(check_cfg(cfg));
  if (!delta) return fail(MOE_ERR_INVALID_ARG, "delta is NULL");
  *delta = cfg->gate == MOE_GATE_SOFTMAX ? kRecheckDeltaSoftmax : kRecheckDeltaSigmoid;
  return MOE_OK;
}

moe_status moe_workspace_size(const moe_config* cfg, size_t* bytes) {
  MOE_TRY(check_cfg(cfg));
  if (!bytes) return fail(MOE_ERR_INVALID_ARG, "bytes is NULL");
  *bytes = layout(cfg).total;
  return MOE_OK;
}

moe_status moe_route(const moe_config* cfg, const moe_layer* layer, const void* u, const float* bias, int32_t* topk_idx,
                     float* topk_w, void* ws, size_t ws_bytes, hipStream_t stream) {
  MOE_TRY(check_cfg(cfg));
  MOE_TRY(check_layer_router(layer));
  if (cfg->T > 0 && (!u || !topk_idx || !topk_w)) return fail(MOE_ERR_INVALID_ARG, "u / topk_idx / topk_w is NULL");
  MOE_TRY(check_aligned16({{"u", u}}));
  uint8_t* base;
  Layout L;
  MOE_TRY(check_ws(cfg, ws, ws_bytes, &base, &L));
  if (cfg->T == 0) return MOE_OK;
  return do_route(cfg, layer, u, bias, topk_idx, topk_w, base, L, stream);
}

moe_status moe_router_logits(const moe_config* cfg, const moe_layer* layer, const void* u, float* z, void* ws,
                             size_t ws_bytes, hipStream_t stream) {
  MOE_TRY(check_cfg(cfg));
  MOE_TRY(check_layer_router(layer));
  if (cfg->T > 0 && (!u || !z)) return fail(MOE_ERR_INVALID_ARG, "u / z is NULL");
  MOE_TRY(check_aligned16({{"u", u}}));
  uint8_t* base;
  Layout L;
  MOE_TRY(check_ws(cfg, ws, ws_bytes, &base, &L));
  RouteArgs a = route_args(cfg, layer, u, nullptr, nullptr, nullptr, base, L);
  a.z = z;
  return hip_status(launch_router_logits(a, stream), "router logits launch");
}

moe_status moe_dispatch(const moe_config* cfg, const int32_t* topk_idx, int32_t* counts, int32_t* offsets,
                        int32_t* perm_src, int32_t* row_of, void* ws, size_t ws_bytes, hipStream_t stream) {
  MOE_TRY(check_cfg(cfg));
  if (!counts || !offsets) return fail(MOE_ERR_INVALID_ARG, "counts / offsets is NULL");
  if (cfg->T > 0 && (!topk_idx || !perm_src || !row_of)) return fail(MOE_ERR_INVALID_ARG, "topk_idx / perm_src / row_of is NULL");
  uint8_t* base;
  Layout L;
  MOE_TRY(check_ws(cfg, ws, ws_bytes, &base, &L));
  if (cfg->T == 0) {
    MOE_TRY(hip_status(launch_zero_fill(counts, sizeof(int32_t) * cfg->n_routed, stream), "counts clear"));
    return hip_status(launch_zero_fill(offsets, sizeof(int32_t) * (cfg->n_routed + 1), stream), "offsets clear");
  }
  return do_dispatch(cfg, topk_idx, counts, offsets, perm_src, row_of, base, L, stream);
}

moe_status moe_expert_ffn(const moe_config* cfg, const moe_layer* layer, const void* u, const int32_t* offsets,
                          const int32_t* perm_src, void* y_routed, void* y_shared, void* ws, size_t ws_bytes,
                          hipStream_t stream) {
  MOE_TRY(check_cfg(cfg));
  MOE_TRY(check_layer_experts(cfg, layer));
  if (cfg->T > 0 && (!u || !offsets || !perm_src || !y_routed)) return fail(MOE_ERR_INVALID_ARG, "u / offsets / perm_src / y_routed is NULL");
  if (cfg->T > 0 && cfg->n_shared > 0 && !y_shared) return fail(MOE_ERR_INVALID_ARG, "y_shared is NULL with n_shared > 0");
  MOE_TRY(check_aligned16({{"u", u}, {"y_routed", y_routed}, {"y_shared", cfg->n_shared > 0 ? y_shared : nullptr}}));
  uint8_t* base;
  Layout L;
  MOE_TRY(check_ws(cfg, ws, ws_bytes, &base, &L));
  return do_ffn(cfg, layer, u, offsets, perm_src, y_routed, cfg->n_shared > 0 ? y_shared : nullptr, base, L, stream);
}

moe_status moe_combine(const moe_config* cfg, const void* u, const void* y_routed, const void* y_shared,
                       const int32_t* row_of, const float* topk_w, void* h, hipStream_t stream) {
  MOE_TRY(check_cfg(cfg));
  if (cfg->T == 0) return MOE_OK;
  if (!u || !y_routed || !row_of || !topk_w || !h) return fail(MOE_ERR_INVALID_ARG, "combine pointer is NULL");
  if (cfg->n_shared > 0 && !y_shared) return fail(MOE_ERR_INVALID_ARG, "y_shared is NULL with n_shared > 0");
  MOE_TRY(check_aligned16({{"u", u}, {"y_routed", y_routed}, {"y_shared", cfg->n_shared > 0 ? y_shared : nullptr}, {"h", h}}));
  const bool bf16 = cfg->act_dtype == MOE_BF16;
  MOE_TRY(hip_status(launch_combine(u, bf16, y_routed, cfg->n_shared > 0 ? y_shared : nullptr, esz_y(cfg) == 2, row_of,
                                    topk_w, cfg->T, cfg->d_model, cfg->top_k, h, stream),
                     "combine launch"));
  mark(MOE_MARK_COMBINE_END, stream);
  return MOE_OK;
}

moe_status moe_forward(const moe_config* cfg, const moe_layer* layer, const void* u, const float* bias, void* h,
                       int32_t* topk_idx, int32_t* counts, void* ws, size_t ws_bytes, hipStream_t stream) {
  MOE_TRY(check_cfg(cfg));
  MOE_TRY(check_layer_router(layer));
  MOE_TRY(check_layer_experts(cfg, layer));
  if (cfg->T > 0 && (!u || !h)) return fail(MOE_ERR_INVALID_ARG, "u / h is NULL");
  MOE_TRY(check_aligned16({{"u", u}, {"h", h}}));
  uint8_t* base;
  Layout L;
  MOE_TRY(check_ws(cfg, ws, ws_bytes, &base, &L));
  int32_t* idx = topk_idx ? topk_idx : reinterpret_cast<int32_t*>(base + L.f_idx);
  int32_t* cnt = counts ? counts : reinterpret_cast<int32_t*>(base + L.f_counts);
  if (cfg->T == 0) {
    if (counts) return hip_status(launch_zero_fill(counts, sizeof(int32_t) * cfg->n_routed, stream), "counts clear");
    return MOE_OK;
  }
  float* w = reinterpret_cast<float*>(base + L.f_w);
  int32_t* offsets = reinterpret_cast<int32_t*>(base + L.f_offsets);
  int32_t* perm = reinterpret_cast<int32_t*>(base + L.f_perm);
  int32_t* row_of = reinterpret_cast<int32_t*>(base + L.f_rowof);
  void* yr = base + L.f_yr;
  void* ys = cfg->n_shared > 0 ? static_cast<void*>(base + L.f_ys) : nullptr;
  MOE_TRY(do_route(cfg, layer, u, bias, idx, w, base, L, stream));
  MOE_TRY(do_dispatch(cfg, idx, cnt, offsets, perm, row_of, base, L, stream));
  MOE_TRY(do_ffn(cfg, layer, u, offsets, perm, yr, ys, base, L, stream));
  MOE_TRY(hip_status(launch_combine(u, cfg->act_dtype == MOE_BF16, yr, ys, esz_y(cfg) == 2, row_of, w, cfg->T,
                                    cfg->d_model, cfg->top_k, h, stream),
                     "combine launch"));
  mark(MOE_MARK_COMBINE_END, stream);
  return MOE_OK;
}

// ------------------------------------------------------------------ allocation-free forward
// Scratch of moe_forward_noalloc: one copy per GPU, held from the library's load on that GPU until the
// process ends. Host code never passes `scratch` itself to a kernel or a copy: it is a host-side stand-in;
// the device address of a GPU's copy comes from hipGetSymbolAddress with that GPU current.
static __device__ __align__(256) uint8_t scratch[MOE_NOALLOC_SCRATCH_BYTES];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// The device address of the current GPU's scratch, looked up once per GPU.
moe_status scratch_of_current_device(void** out) {
  int dev = -1;
  MOE_TRY(hip_status(hipGetDevice(&dev), "hipGetDevice"));
  if (dev < 0 || dev >= kMaxDevices) return fail(MOE_ERR_UNSUPPORTED, "device %d: at most %d devices", dev, kMaxDevices);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    MOE_TRY(hip_status(hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)), "hipGetSymbolAddress(scratch)"));
    if (!p) return fail(MOE_ERR_HIP, "hipGetSymbolAddress(scratch) returned NULL");
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return MOE_OK;
}
}  // namespace

moe_status moe_forward_noalloc(const moe_config* cfg, const moe_layer* layer, const void* u, const float* bias, void* h,
                               int32_t* topk_idx, int32_t* counts, hipStream_t stream) {
  MOE_TRY(check_cfg(cfg));
  const size_t need = layout(cfg).total;
  if (need > (size_t)MOE_NOALLOC_SCRATCH_BYTES)
    return fail(MOE_ERR_WORKSPACE,
                "moe_forward_noalloc: this configuration needs %zu bytes of scratch, above the library's static %zu "
                "(use moe_forward with a workspace)",
                need, (size_t)MOE_NOALLOC_SCRATCH_BYTES);
  void* ws = nullptr;
  MOE_TRY(scratch_of_current_device(&ws));
  return moe_forward(cfg, layer, u, bias, h, topk_idx, counts, ws, (size_t)MOE_NOALLOC_SCRATCH_BYTES, stream);
}

moe_status moe_update_bias(const moe_config* cfg, const int32_t* counts, float gamma, float* bias, hipStream_t stream) {
  MOE_TRY(check_cfg(cfg));
  if (!counts || !bias) return fail(MOE_ERR_INVALID_ARG, "counts / bias is NULL");
  return hip_status(launch_bias_update(counts, cfg->n_routed, (long long)cfg->T * cfg->top_k, gamma, bias, stream),
                    "bias update launch");
}

moe_status moe_balance_stats(const moe_config* cfg, const float* z, const int32_t* topk_idx, int32_t seq_len,
                             float alpha_expert, float alpha_seq, float* f, float* P, float* loss, void* ws,
                             size_t ws_bytes, hipStream_t stream) {
  MOE_TRY(check_cfg(cfg));
  if (seq_len <= 0 || cfg->T % seq_len)
    return fail(MOE_ERR_INVALID_ARG, "seq_len=%d must be positive and divide T=%d", seq_len, cfg->T);
  if (seq_len != cfg->T && seq_len % 64)
    return fail(MOE_ERR_UNSUPPORTED, "seq_len=%d must equal T or be a multiple of 64", seq_len);
  if (cfg->T > 0 && (!z || !topk_idx || !f || !P || !loss)) return fail(MOE_ERR_INVALID_ARG, "z / topk_idx / f / P / loss is NULL");
  uint8_t* base;
  Layout L;
  MOE_TRY(check_ws(cfg, ws, ws_bytes, &base, &L));
  BalanceArgs a{};
  a.z = z;
  a.idx = topk_idx;
  a.T = cfg->T;
  a.E = cfg->n_routed;
  a.K = cfg->top_k;
  a.gate = cfg->gate;
  a.seq_len = seq_len;
  a.alpha_expert = alpha_expert;
  a.alpha_seq = alpha_seq;
  a.psum = reinterpret_cast<double*>(base + L.bal_psum);
  a.cnt = reinterpret_cast<int32_t*>(base + L.bal_cnt);
  a.seq_p = reinterpret_cast<double*>(base + L.bal_seqp);
  a.seq_n = reinterpret_cast<int32_t*>(base + L.bal_seqn);
  a.seq_term = reinterpret_cast<double*>(base + L.bal_seq);
  a.f = f;
  a.P = P;
  a.loss = loss;
  return hip_status(launch_balance_stats(a, stream), "balance statistics launch");
}

moe_status moe_backward_workspace_size(const moe_config* cfg, size_t* bytes) {
  MOE_TRY(check_bwd_cfg(cfg));
  if (!bytes) return fail(MOE_ERR_INVALID_ARG, "bytes is NULL");
  *bytes = bwd_layout(cfg).total;
  return MOE_OK;
}

moe_status moe_pack_weights(const moe_config* cfg, int32_t which, const void* src, void* dst, hipStream_t stream) {
  MOE_TRY(check_cfg(cfg));
  if (cfg->w_dtype == MOE_F32) return fail(MOE_ERR_UNSUPPORTED, "the tiled weight layout is for bf16 and fp8 weights");
  const int esz = cfg->w_dtype == MOE_FP8_E4M3 ? 1 : 2;
  const int E = cfg->n_routed, d = cfg->d_model, f = cfg->inter_dim, fs = cfg->n_shared * f;
  int groups = 0, rows = 0, cols = 0;
  bool gateup = false;
  switch (which) {
    case MOE_PACK_W13: groups = E; rows = 2 * f; cols = d; gateup = true; break;
    case MOE_PACK_W2: groups = E; rows = d; cols = f; break;
    case MOE_PACK_WS13: groups = fs > 0 ? 1 : 0; rows = 2 * fs; cols = d; gateup = true; break;
    case MOE_PACK_WS2: groups = fs > 0 ? 1 : 0; rows = d; cols = fs; break;
    case MOE_PACK_W13T: groups = E; rows = d; cols = 2 * f; break;
    case MOE_PACK_W2T: groups = E; rows = f; cols = d; break;
    case MOE_PACK_WS13T: groups = fs > 0 ? 1 : 0; rows = d; cols = 2 * fs; break;
    case MOE_PACK_WS2T: groups = fs > 0 ? 1 : 0; rows = fs; cols = d; break;
    default: return fail(MOE_ERR_INVALID_ARG, "bad which %d", which);
  }
  if (groups == 0) return MOE_OK;
  if (rows % 256) return fail(MOE_ERR_UNSUPPORTED, "the matrix has %d rows, not a multiple of 256", rows);
  if (!src || !dst) return fail(MOE_ERR_INVALID_ARG, "src / dst is NULL");
  if (src == dst) return fail(MOE_ERR_INVALID_ARG, "the layout change cannot run in place");
  MOE_TRY(check_aligned16({{"src", src}, {"dst", dst}}));
  // check_cfg has d % 256 == 0 and f % 128 == 0: gate/up tiles of 128 + 128 rows, down tiles of 256 rows,
  // 128-byte K stages
  return hip_status(launch_pack_weights(src, dst, groups, rows, cols * esz, gateup, stream), "weight layout launch");
}

moe_status moe_transpose_fp8_weights(const uint8_t* q, const float* scales, int32_t batch, int32_t rows, int32_t cols,
                                     uint8_t* qt, float* scales_t, hipStream_t stream) {
  if (batch < 0 || rows <= 0 || cols <= 0) return fail(MOE_ERR_INVALID_ARG, "bad sizes batch=%d rows=%d cols=%d", batch, rows, cols);
  if (rows % 128 || cols % 128) return fail(MOE_ERR_UNSUPPORTED, "rows and cols must be multiples of 128");
  if (batch > 65535 || rows / 64 > 65535) return fail(MOE_ERR_UNSUPPORTED, "too many blocks");
  if (batch > 0 && (!q || !scales || !qt || !scales_t)) return fail(MOE_ERR_INVALID_ARG, "q / scales / qt / scales_t is NULL");
  MOE_TRY(check_aligned16({{"q", q}, {"qt", qt}}));
  return hip_status(launch_transpose_fp8(q, scales, batch, rows, cols, qt, scales_t, stream), "weight transpose launch");
}

moe_status moe_expert_ffn_backward(const moe_config* cfg, const moe_layer* layer, const moe_layer* layer_t,
                                   const void* u, const int32_t* offsets, const int32_t* perm_src, const void* dy_routed,
                                   const void* dy_shared, void* dx_routed, void* dx_shared, void* dw13, void* dw2,
                                   void* dws13, void* dws2, void* ws, size_t ws_bytes, hipStream_t stream) {
  MOE_TRY(check_bwd_cfg(cfg));
  MOE_TRY(check_layer_experts(cfg, layer));
  MOE_TRY(check_layer_experts(cfg, layer_t));
  const moe_config* c = cfg;
  const bool sh = c->n_shared > 0;
  const bool want_dx = dx_routed != nullptr, want_dw = dw13 != nullptr;
  if (!want_dx && !want_dw) return fail(MOE_ERR_INVALID_ARG, "neither dx_routed nor dw13 is given");
  if (want_dw && !dw2) return fail(MOE_ERR_INVALID_ARG, "dw2 is NULL while dw13 is given");
  if (want_dw && sh && (!dws13 || !dws2)) return fail(MOE_ERR_INVALID_ARG, "dws13 / dws2 is NULL with n_shared > 0");
  if (c->T > 0 && (!u || !offsets || !perm_src || !dy_routed))
    return fail(MOE_ERR_INVALID_ARG, "u / offsets / perm_src / dy_routed is NULL");
  if (c->T > 0 && sh && !dy_shared) return fail(MOE_ERR_INVALID_ARG, "dy_shared is NULL with n_shared > 0");
  if (want_dx && c->T > 0 && sh && !dx_shared) return fail(MOE_ERR_INVALID_ARG, "dx_shared is NULL with n_shared > 0");
  MOE_TRY(check_aligned16({{"u", u}, {"dy_routed", dy_routed}, {"dy_shared", sh ? dy_shared : nullptr},
                           {"dx_routed", dx_routed}, {"dx_shared", sh ? dx_shared : nullptr}, {"dw13", dw13},
                           {"dw2", dw2}, {"dws13", sh ? dws13 : nullptr}, {"dws2", sh ? dws2 : nullptr}}));
  const BwdLayout L = bwd_layout(c);
  if (!ws) return fail(MOE_ERR_WORKSPACE, "workspace is NULL");
  if (ws_bytes < L.total) return fail(MOE_ERR_WORKSPACE, "workspace %zu bytes < required %zu", ws_bytes, L.total);
  if (c->T == 0) {
    // no rows: every weight gradient is zero
    if (want_dw) {
      const size_t n13 = (size_t)c->n_routed * 2 * c->inter_dim * c->d_model * 2, n2 = n13 / 2;
      MOE_TRY(hip_status(launch_zero_fill(dw13, n13, stream), "weight gradient clear"));
      MOE_TRY(hip_status(launch_zero_fill(dw2, n2, stream), "weight gradient clear"));
      if (sh) {
        const size_t s13 = (size_t)2 * c->inter_dim * c->d_model * 2;
        MOE_TRY(hip_status(launch_zero_fill(dws13, s13, stream), "weight gradient clear"));
        MOE_TRY(hip_status(launch_zero_fill(dws2, s13 / 2, stream), "weight gradient clear"));
      }
    }
    return MOE_OK;
  }
  uint8_t* base = reinterpret_cast<uint8_t*>(align_up(reinterpret_cast<uintptr_t>(ws), 256));
  hipStream_t s = stream;
  const int T = c->T, E = c->n_routed, d = c->d_model, f = c->inter_dim, fs = c->n_shared * f;
  const int rows = T * c->top_k;
  const int bm = gemm_mfma_bm(), grid = device_cus() / 8 * 8;
  auto F = [&](size_t o) { return reinterpret_cast<float*>(base + o); };
  int32_t* mt_prefix = reinterpret_cast<int32_t*>(base + L.mt_prefix);
  int32_t* xa = reinterpret_cast<int32_t*>(base + L.xsched_a);
  int32_t* xb = reinterpret_cast<int32_t*>(base + L.xsched_b);
  // tile ranges: (g, v) recompute [gate/up shape] and da = dy W2 [down shape, output f]; then dx [output d]
  {
    const int nt_r[2] = {f / 128, f / 256}, nt_s[2] = {fs / 128, sh ? f / 256 : 0};
    MOE_TRY(hip_status(launch_schedule_mfma(offsets, E, T, bm, nt_r, nt_s, mt_prefix, xa, xa + 2 * kSchedRange, s), "schedule launch"));
    const int nt_r2[2] = {f / 128, d / 256}, nt_s2[2] = {0, sh ? d / 256 : 0};
    MOE_TRY(hip_status(launch_schedule_mfma(offsets, E, T, bm, nt_r2, nt_s2, mt_prefix, xb, xb + 2 * kSchedRange, s), "schedule launch"));
  }
  // cached forward input: u quantized 1x128 as in the forward
  MOE_TRY(hip_status(launch_quant_act(u, true, T, d, base + L.uq, F(L.us), s), "activation quantization launch"));
  GemmArgs g{};
  g.E = E;
  g.T = T;
  g.offsets = offsets;
  g.perm_src = perm_src;
  g.mt_prefix = mt_prefix;
  // 1. [g | v] = x [W1; W3]^T in fp32 (the forward's gate/up GEMM without SwiGLU)
  g.d = d;
  g.f = f;
  g.fs = fs;
  g.xrange = xa;
  g.xcount = xa + 2 * kSchedRange;
  g.w_routed = static_cast<const uint8_t*>(layer->w13);
  g.w_shared = static_cast<const uint8_t*>(layer->ws13);
  g.ws_routed = layer->w13_scale;
  g.ws_shared = layer->ws13_scale;
  g.x_routed = g.x_shared = base + L.uq;
  g.xs_routed = g.xs_shared = F(L.us);
  g.out_routed = base + L.gv_r;
  g.out_shared = base + L.gv_s;
  g.packed = layer->weight_layout == MOE_LAYOUT_TILED;
  MOE_TRY(hip_status(launch_gemm_mfma(g, true, true, grid, s, true), "g/v GEMM launch"));
  g.packed = layer_t->weight_layout == MOE_LAYOUT_TILED;   // the transposed weights below
  // 2. dy quantized 1x128 along d; da = dy W2 (weights W2^T [f, d]: output f, contraction d), fp32
  MOE_TRY(hip_status(launch_quant_act(dy_routed, true, rows, d, base + L.dyq_r, F(L.dys_r), s), "dy quantization launch"));
  if (sh) MOE_TRY(hip_status(launch_quant_act(dy_shared, true, T, d, base + L.dyq_s, F(L.dys_s), s), "dy quantization launch"));
  g.d = f;
  g.f = d;
  g.fs = d;
  g.xrange = xa + kSchedRange;
  g.xcount = xa + 2 * kSchedRange + kSchedCount;
  g.w_routed = static_cast<const uint8_t*>(layer_t->w2);
  g.w_shared = static_cast<const uint8_t*>(layer_t->ws2);
  g.ws_routed = layer_t->w2_scale;
  g.ws_shared = layer_t->ws2_scale;
  g.x_routed = base + L.dyq_r;
  g.x_shared = base + L.dyq_s;
  g.xs_routed = F(L.dys_r);
  g.xs_shared = F(L.dys_s);
  g.out_routed = base + L.da_r;
  g.out_shared = base + L.da_s;
  MOE_TRY(hip_status(launch_gemm_mfma(g, true, false, grid, s, true), "da GEMM launch"));
  if (want_dw) MOE_TRY(weight_gradients(c, L, base, u, offsets, perm_src, dy_routed, dy_shared, dw13, dw2, dws13, dws2, s));
  if (!want_dx) return MOE_OK;
  // 3. [dg | dv] from da, g, v, quantized 1x128 along 2f
  MOE_TRY(hip_status(launch_swiglu_backward_quant(F(L.da_r), F(L.gv_r), rows, f, base + L.dgq_r, F(L.dgs_r), s),
                     "SwiGLU backward launch"));
  if (sh)
    MOE_TRY(hip_status(launch_swiglu_backward_quant(F(L.da_s), F(L.gv_s), T, fs, base + L.dgq_s, F(L.dgs_s), s),
                       "SwiGLU backward launch"));
  // 4. dx = [dg | dv] [W1; W3] (weights [W1; W3]^T [d, 2f]: output d, contraction 2f), bf16
  g.d = d;
  g.f = 2 * f;
  g.fs = 2 * fs;
  g.xrange = xb + kSchedRange;
  g.xcount = xb + 2 * kSchedRange + kSchedCount;
  g.w_routed = static_cast<const uint8_t*>(layer_t->w13);
  g.w_shared = static_cast<const uint8_t*>(layer_t->ws13);
  g.ws_routed = layer_t->w13_scale;
  g.ws_shared = layer_t->ws13_scale;
  g.x_routed = base + L.dgq_r;
  g.x_shared = base + L.dgq_s;
  g.xs_routed = F(L.dgs_r);
  g.xs_shared = F(L.dgs_s);
  g.out_routed = static_cast<uint8_t*>(dx_routed);
  g.out_shared = static_cast<uint8_t*>(dx_shared);
  MOE_TRY(hip_status(launch_gemm_mfma(g, true, false, grid, s, false), "dx GEMM launch"));
  return MOE_OK;
}

moe_status moe_expert_ffn_backward_input(const moe_config* cfg, const moe_layer* layer, const moe_layer* layer_t,
                                         const void* u, const int32_t* offsets, const int32_t* perm_src,
                                         const void* dy_routed, const void* dy_shared, void* dx_routed, void* dx_shared,
                                         void* ws, size_t ws_bytes, hipStream_t stream) {
  if (!dx_routed && cfg && cfg->T > 0) return fail(MOE_ERR_INVALID_ARG, "dx_routed is NULL");
  if (!dx_routed) return check_bwd_cfg(cfg);
  return moe_expert_ffn_backward(cfg, layer, layer_t, u, offsets, perm_src, dy_routed, dy_shared, dx_routed, dx_shared,
                                 nullptr, nullptr, nullptr, nullptr, ws, ws_bytes, stream);
}

moe_status moe_quantize_weights(const float* w, int32_t batch, int32_t rows, int32_t cols, uint8_t* q, float* scales,
                                hipStream_t stream) {
  if (batch < 0 || rows <= 0 || cols <= 0) return fail(MOE_ERR_INVALID_ARG, "bad sizes batch=%d rows=%d cols=%d", batch, rows, cols);
  if (rows % 128 || cols % 128) return fail(MOE_ERR_UNSUPPORTED, "rows and cols must be multiples of 128");
  if (batch > 65535 || rows / 128 > 65535) return fail(MOE_ERR_UNSUPPORTED, "too many blocks");
  if (batch > 0 && (!w || !q || !scales)) return fail(MOE_ERR_INVALID_ARG, "w / q / scales is NULL");
  MOE_TRY(check_aligned16({{"w", w}, {"q", q}}));
  return hip_status(launch_quant_weight(w, batch, rows, cols, q, scales, stream), "weight quantization launch");
}

moe_status moe_quantize_act(const void* x, int32_t x_dtype, int32_t rows, int32_t cols, uint8_t* q, float* scales,
                            hipStream_t stream) {
  if (rows < 0 || cols <= 0) return fail(MOE_ERR_INVALID_ARG, "bad sizes rows=%d cols=%d", rows, cols);
  if (x_dtype != MOE_F32 && x_dtype != MOE_BF16) return fail(MOE_ERR_INVALID_ARG, "x_dtype must be F32 or BF16");
  if (cols % 128) return fail(MOE_ERR_UNSUPPORTED, "cols must be a multiple of 128");
  if (rows > 0 && (!x || !q || !scales)) return fail(MOE_ERR_INVALID_ARG, "x / q / scales is NULL");
  MOE_TRY(check_aligned16({{"x", x}, {"q", q}}));
  return hip_status(launch_quant_act(x, x_dtype == MOE_BF16, rows, cols, q, scales, stream), "activation quantization launch");
}

}  // extern "C"
