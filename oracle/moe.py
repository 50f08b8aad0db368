"""DeepSeekMoE layer forward, float64, in the order and notation of the pages.

Notation: T tokens u_t of width d; E routed experts with inner dim f; Ks shared experts, concatenated
into one SwiGLU block of inner dim Ks*f (the sum of Ks FFNs with no gate equals one FFN over the
concatenated inner dim); K routed experts per token.

Readings taken where the pages are silent or disagree (each is repeated where it is used):
* SwiGLU is named but not written out ([PW] "invariant core"): FFN(x) = W2 (SiLU(W1 x) * (W3 x)),
  SiLU(z) = z * sigmoid(z), no biases.
* Softmax gating runs over the routed experts only, and its gates are not renormalised ([TR] §2.3).
* Sigmoid gating ([TR] §3.3, §5.3 [3]-[4]): the bias enters only the selection key s + b; the gate
  comes from the raw s, renormalised over the selected experts when ``renorm`` is set. [YJ] §4.3.2
  writes softmax(score + b) as the gate, which contradicts its own next paragraph and [TR]; not used.
* Top-K ties go to the lower expert index; the selected set is returned in ascending expert order.
* No capacity factor and no token dropping (the pages mention neither).
"""
from __future__ import annotations

import numpy as np

from . import quant


# ----------------------------------------------------------------------------------------- router
def router_logits(u, w_gate, logit_offset=None) -> np.ndarray:
    """z[t, e] = u_t^T e_i ([TR] §2.3 gate, §3.3 affinity), plus an optional per-expert offset."""
    z = np.asarray(u, dtype=np.float64) @ np.asarray(w_gate, dtype=np.float64).T
    if logit_offset is not None:
        z = z + np.asarray(logit_offset, dtype=np.float64)[None, :]
    return z


def softmax(z) -> np.ndarray:
    """g_{i,t} = Softmax_i(z): exp(z - max z) / sum exp(z - max z) over the routed experts."""
    z = np.asarray(z, dtype=np.float64)
    ez = np.exp(z - z.max(axis=1, keepdims=True))
    return ez / ez.sum(axis=1, keepdims=True)


def sigmoid(z) -> np.ndarray:
    """s_{i,t} = Sigmoid(u_t^T e_i) = 1 / (1 + exp(-z)), [TR] §3.3 and §5.3 [3]."""
    with np.errstate(over="ignore"):
        return 1.0 / (1.0 + np.exp(-np.asarray(z, dtype=np.float64)))


def topk_select(key, K: int):
    """Indices of the K largest keys per row under (key descending, index ascending).

    Returns (idx [T, K] int32 in ascending expert order, gap [T]) where gap is the K-th largest key
    minus the (K+1)-th (inf when K == E): the margin by which the selection is decided.
    """
    key = np.asarray(key, dtype=np.float64)
    T, E = key.shape
    order = np.argsort(-key, axis=1, kind="stable")   # stable: equal keys keep ascending index
    idx = np.sort(order[:, :K], axis=1).astype(np.int32)
    if K < E:
        rows = np.arange(T)
        gap = key[rows, order[:, K - 1]] - key[rows, order[:, K]]
    else:
        gap = np.full(T, np.inf)
    return idx, gap


def group_limit(key, n_groups: int, topk_groups: int):
    """Device/node-limited routing ([TR] §2.3 device-limited routing, M = 3 devices; §3.2 and §3.8
    node-limited routing, M = 4 nodes): a token's experts come from at most M groups.

    Reading (the pages do not print the rule): the E experts form n_groups equal contiguous groups
    (group of expert e = e // (E / n_groups)); a group's score is the largest key among its experts;
    the M = topk_groups groups with the largest scores are kept (ties to the lower group index) and
    the keys of every other group are masked to -inf before the top-K.
    Returns (masked key [T, E], group gap [T]): the M-th largest group score minus the (M+1)-th
    (inf when M == n_groups), the margin by which the group choice is decided.
    """
    key = np.asarray(key, dtype=np.float64)
    T, E = key.shape
    gsz = E // n_groups
    gscore = key.reshape(T, n_groups, gsz).max(axis=2)
    order = np.argsort(-gscore, axis=1, kind="stable")     # stable: equal scores keep ascending group
    keep = np.zeros((T, n_groups), dtype=bool)
    np.put_along_axis(keep, order[:, :topk_groups], True, axis=1)
    masked = np.where(np.repeat(keep, gsz, axis=1), key, -np.inf)
    if topk_groups < n_groups:
        rows = np.arange(T)
        ggap = gscore[rows, order[:, topk_groups - 1]] - gscore[rows, order[:, topk_groups]]
    else:
        ggap = np.full(T, np.inf)
    return masked, ggap


def route(z, gate: str, K: int, bias=None, renorm: bool = False, n_groups: int = 0, topk_groups: int = 0):
    """Selection and gates from the logits z [T, E].

    softmax ([TR] §2.3): p = Softmax(z); the K largest p are selected (p is monotone in z, so the key
    is z itself, which avoids ties created by rounding exp); gates g = p of the selected experts.
    sigmoid_bias ([TR] §3.3): s = Sigmoid(z); selected iff s_i + b_i is among the K largest of
    {s_j + b_j}; g' = s of the selected experts; g = g' / sum g' when renorm.
    With n_groups > 0 the selection is first limited to topk_groups groups (group_limit); the gates are
    computed as without the limit.
    Returns dict(idx [T,K] int32 ascending, w [T,K] float64, gap [T], key [T,E], score [T,E]); gap is
    the smaller of the top-K margin and the group margin.
    """
    z = np.asarray(z, dtype=np.float64)
    if gate == "softmax":
        score = softmax(z)
        key = z
    elif gate == "sigmoid_bias":
        score = sigmoid(z)
        b = np.zeros(z.shape[1]) if bias is None else np.asarray(bias, dtype=np.float64)
        key = score + b[None, :]
    else:
        raise ValueError(gate)
    if n_groups:
        if z.shape[1] % n_groups or not 1 <= topk_groups <= n_groups or K > topk_groups * (z.shape[1] // n_groups):
            raise ValueError("bad group limit")
        masked, ggap = group_limit(key, n_groups, topk_groups)
        idx, gap = topk_select(masked, K)
        gap = np.minimum(gap, ggap)
    else:
        idx, gap = topk_select(key, K)
    w = np.take_along_axis(score, idx.astype(np.int64), axis=1)
    if renorm:
        w = w / w.sum(axis=1, keepdims=True)
    return dict(idx=idx, w=w, gap=gap, key=key, score=score)


def expert_counts(idx, E: int) -> np.ndarray:
    """Number of tokens that selected each routed expert (the load of [TR] §3.3)."""
    return np.bincount(np.asarray(idx).reshape(-1), minlength=E).astype(np.int32)


# --------------------------------------------------------------------------------------- dispatch
def dispatch(idx, E: int):
    """Group the (token, slot) pairs by expert, tokens ascending inside each expert.

    Returns offsets [E+1] (exclusive prefix sum of the counts), perm_src [T*K] (token of each
    expert-ordered row) and row_of [T, K] (row of each pair), all int32.
    """
    idx = np.asarray(idx)
    T, K = idx.shape
    counts = expert_counts(idx, E)
    offsets = np.zeros(E + 1, dtype=np.int64)
    offsets[1:] = np.cumsum(counts)
    perm_src = np.empty(T * K, dtype=np.int32)
    row_of = np.empty((T, K), dtype=np.int32)
    fill = offsets[:-1].copy()
    for t in range(T):                                  # tokens in ascending order
        for k in range(K):
            e = idx[t, k]
            perm_src[fill[e]] = t
            row_of[t, k] = fill[e]
            fill[e] += 1
    return offsets.astype(np.int32), perm_src, row_of


# -------------------------------------------------------------------------------------- experts
def silu(z) -> np.ndarray:
    with np.errstate(over="ignore"):
        return z / (1.0 + np.exp(-z))


def swiglu_ffn(x, w1, w3, w2) -> np.ndarray:
    """FFN(x) = W2 (SiLU(W1 x) * (W3 x)) for each row of x, float64 ([PW] "invariant core")."""
    x = np.asarray(x, dtype=np.float64)
    g = x @ np.asarray(w1, dtype=np.float64).T
    v = x @ np.asarray(w3, dtype=np.float64).T
    return (silu(g) * v) @ np.asarray(w2, dtype=np.float64).T


def swiglu_ffn_fp8(x, w13q, w13s, w2q, w2s) -> tuple[np.ndarray, np.ndarray]:
    """The SwiGLU expert with every Linear forward GEMM in E4M3, [TR] §3.6.

    x [rows, d] is quantized 1x128, multiplied with the 128x128-block-quantized [W1; W3]
    (w13q [2f, d], W1 rows first) with per-128 promotion, SiLU(g) * v is formed in float64, rounded
    to fp32, quantized 1x128 again, and multiplied with W2 (w2q [d, f]) the same way.
    Returns (y [rows, d] float64, a [rows, f] float64 before its requantization).
    """
    f = w13q.shape[0] // 2
    xq, xs = quant.quantize_act_1x128(x)
    gv = quant.gemm_blockscaled(xq, xs, w13q, w13s)
    a = silu(gv[:, :f]) * gv[:, f:]
    aq, as_ = quant.quantize_act_1x128(a.astype(np.float32))
    y = quant.gemm_blockscaled(aq, as_, w2q, w2s)
    return y, a


# ------------------------------------------------------------------------- expert backward (input)
def swiglu_backward(da, g, v):
    """Gradients of a = SiLU(g) * v with respect to g and v for the upstream gradient da (float64):
    dv = da * SiLU(g), dg = da * v * SiLU'(g), SiLU'(g) = sigmoid(g) * (1 + g * (1 - sigmoid(g)))."""
    da, g, v = (np.asarray(t, dtype=np.float64) for t in (da, g, v))
    sig = sigmoid(g)
    return da * v * sig * (1.0 + g * (1.0 - sig)), da * g * sig


def swiglu_ffn_backward_input(dy, x, w1, w3, w2) -> np.ndarray:
    """dx of FFN(x) = W2 (SiLU(W1 x) * (W3 x)) for the row gradients dy, float64 (the chain rule through
    the three Linears and SwiGLU; [PW] "invariant core" for the FFN)."""
    x = np.asarray(x, dtype=np.float64)
    w1, w3, w2 = (np.asarray(w, dtype=np.float64) for w in (w1, w3, w2))
    g, v = x @ w1.T, x @ w3.T
    dg, dv = swiglu_backward(np.asarray(dy, dtype=np.float64) @ w2, g, v)
    return dg @ w1 + dv @ w3


def swiglu_ffn_backward_input_fp8(dy, x, w13q, w13s, w2q, w2s) -> np.ndarray:
    """The activation backward GEMMs of the SwiGLU expert in E4M3 ([TR] §3.6: the GEMMs of the
    activation gradients run in FP8, 1x128 activation tiles, 128x128 weight blocks, promotion every 128).

    Readings (the pages fix the formats, not the dataflow): the cached forward input x is quantized
    1x128 as in the forward and g, v are recomputed from it with the forward GEMM; the output gradient
    dy is quantized 1x128 along d, the contraction of da = dy W2; the SwiGLU backward is evaluated and
    rounded to fp32; [dg | dv] is quantized 1x128 along 2f, the contraction of dx = [dg | dv] [W1; W3].
    A transposed weight keeps its E4M3 codes and the transposed grid of 128x128 block scales.
    """
    f = w13q.shape[0] // 2
    xq, xs = quant.quantize_act_1x128(x)
    gv = quant.gemm_blockscaled(xq, xs, w13q, w13s)
    dyq, dys = quant.quantize_act_1x128(np.asarray(dy).astype(np.float32))
    da = quant.gemm_blockscaled(dyq, dys, np.ascontiguousarray(w2q.T), np.ascontiguousarray(w2s.T))
    dg, dv = swiglu_backward(da, gv[:, :f], gv[:, f:])
    dgvq, dgvs = quant.quantize_act_1x128(np.hstack([dg, dv]).astype(np.float32))
    return quant.gemm_blockscaled(dgvq, dgvs, np.ascontiguousarray(w13q.T), np.ascontiguousarray(w13s.T))


# ------------------------------------------------------------------------ expert backward (weights)
def swiglu_ffn_backward_weight(dy, x, w1, w3, w2):
    """(dW1, dW3, dW2) of FFN(x) = W2 (SiLU(W1 x) * (W3 x)) summed over the rows of x for the row
    gradients dy, float64: dW2 = dy^T a with a = SiLU(g) * v, dW1 = dg^T x, dW3 = dv^T x."""
    x, dy = np.asarray(x, dtype=np.float64), np.asarray(dy, dtype=np.float64)
    w1, w3, w2 = (np.asarray(w, dtype=np.float64) for w in (w1, w3, w2))
    g, v = x @ w1.T, x @ w3.T
    dg, dv = swiglu_backward(dy @ w2, g, v)
    return dg.T @ x, dv.T @ x, dy.T @ (silu(g) * v)


def swiglu_ffn_backward_weight_fp8(dy, x, w13q, w13s, w2q, w2s, operands: bool = False):
    """The weight-gradient GEMMs of the SwiGLU expert in E4M3 ([TR] §3.6: the weight backward GEMM runs
    in FP8, activations cached for the backward are FP8, weight gradients are kept in BF16).

    Readings: the contraction of dW2 = dy^T a and of d[W1; W3] = [dg | dv]^T x is over the rows
    (tokens), so both operands are quantized in 1x128 tiles along the rows (quant.quantize_act_along_rows;
    an expert's last tile is padded with zero rows). The cached activations enter as the values their
    forward E4M3 copies hold: x as its 1x128 quantization along d, a = SiLU(g) * v as its 1x128
    requantization along f, each dequantized (rounded to fp32) and requantized along the rows. dy enters
    as given, [dg | dv] as its fp32 value from the input backward (swiglu_ffn_backward_input_fp8).
    Returns (dW13 [2f, d] with the W1 rows first, dW2 [d, f]) in float64, before the BF16 rounding; with
    ``operands`` also a dict of the quantizer inputs and outputs (for tests that bound rounding flips).
    """
    f = w13q.shape[0] // 2
    xq, xs = quant.quantize_act_1x128(x)
    gv = quant.gemm_blockscaled(xq, xs, w13q, w13s)
    g, v = gv[:, :f], gv[:, f:]
    aq, as_ = quant.quantize_act_1x128((silu(g) * v).astype(np.float32))
    dy32 = np.asarray(dy).astype(np.float32)
    dyq, dys = quant.quantize_act_1x128(dy32)
    da = quant.gemm_blockscaled(dyq, dys, np.ascontiguousarray(w2q.T), np.ascontiguousarray(w2s.T))
    dg, dv = swiglu_backward(da, g, v)
    dgv = np.hstack([dg, dv]).astype(np.float32)
    a_deq = quant.dequant_act(aq, as_).astype(np.float32)
    x_deq = quant.dequant_act(xq, xs).astype(np.float32)
    dy_t, a_t = quant.quantize_act_along_rows(dy32), quant.quantize_act_along_rows(a_deq)
    dgv_t, x_t = quant.quantize_act_along_rows(dgv), quant.quantize_act_along_rows(x_deq)
    dw2 = quant.gemm_rowscaled(*dy_t, *a_t)
    dw13 = quant.gemm_rowscaled(*dgv_t, *x_t)
    if operands:
        return dw13, dw2, dict(a32=(silu(g) * v).astype(np.float32), a_fwd=(aq, as_), a_deq=a_deq, a_t=a_t,
                               dy_t=dy_t, dgv32=dgv, dgv_t=dgv_t, x_deq=x_deq, x_t=x_t)
    return dw13, dw2


# -------------------------------------------------------------------------------------- combine
def combine(u, y_shared, y_rows, row_of, w) -> np.ndarray:
    """h_t = u_t + sum_shared FFN(u_t) + sum_k g_{k,t} FFN_{e_k}(u_t) ([TR] §1.1, §5.3 [1]).

    Summed in float64 left to right: u, then the shared output, then the routed terms in ascending
    expert order (the order of row_of's columns).
    """
    h = np.asarray(u, dtype=np.float64) + np.asarray(y_shared, dtype=np.float64)
    for k in range(row_of.shape[1]):
        h = h + w[:, k:k + 1] * y_rows[row_of[:, k]]
    return h


# ----------------------------------------------------------------------------------- bias update
def bias_update(bias, counts, gamma: float, T: int, K: int) -> np.ndarray:
    """b_i <- b_i - gamma if expert i is overloaded, b_i + gamma if underloaded ([TR] §3.3).

    Overloaded / underloaded is read as load above / below the mean load T*K/E, decided in integers
    (c_i * E against T*K); a load equal to the mean leaves b_i unchanged. The update is one fp32
    subtraction of gamma * sign.
    """
    b = np.asarray(bias, dtype=np.float32)
    c = np.asarray(counts, dtype=np.int64)
    E = b.shape[0]
    sign = np.sign(c * E - T * K).astype(np.float32)
    return (b - np.float32(gamma) * sign).astype(np.float32)


# ---------------------------------------------------------------------------------------- layer
def layer_forward(u, w_gate, experts, shared, *, gate: str, K: int, bias=None, renorm=False,
                  logit_offset=None, fp8=False, n_groups: int = 0, topk_groups: int = 0):
    """The whole layer. ``experts[e]`` and ``shared`` are the expert weights:

    float path: (w1 [f, d], w3 [f, d], w2 [d, f]) as stored (fp32 or bf16 values);
    fp8 path:   (w13q [2f, d] uint8, w13s [2f/128, d/128], w2q [d, f] uint8, w2s [d/128, f/128]).
    Returns a dict with h, the routing, the per-row expert outputs y_rows (expert-ordered), the
    shared output and the routed sum.
    """
    u = np.asarray(u, dtype=np.float64)
    T = u.shape[0]
    E = len(experts)
    z = router_logits(u, w_gate, logit_offset)
    r = route(z, gate, K, bias, renorm, n_groups, topk_groups)
    offsets, perm_src, row_of = dispatch(r["idx"], E)
    ffn = (lambda x, p: swiglu_ffn_fp8(x, *p)[0]) if fp8 else (lambda x, p: swiglu_ffn(x, *p))
    d = u.shape[1]
    y_rows = np.zeros((T * K, d), dtype=np.float64)
    for e in range(E):
        a, b = offsets[e], offsets[e + 1]
        if b > a:
            y_rows[a:b] = ffn(u[perm_src[a:b]], experts[e])
    y_shared = ffn(u, shared) if shared is not None else np.zeros_like(u)
    h = combine(u, y_shared, y_rows, row_of, r["w"])
    routed = combine(np.zeros_like(u), np.zeros_like(u), y_rows, row_of, r["w"])
    return dict(h=h, z=z, idx=r["idx"], w=r["w"], gap=r["gap"], counts=expert_counts(r["idx"], E),
                offsets=offsets, perm_src=perm_src, row_of=row_of, y_rows=y_rows, y_shared=y_shared,
                routed=routed)


def layer_forward_dense(u, w_gate, experts, shared, *, gate: str, K: int, bias=None, renorm=False,
                        logit_offset=None, fp8=False) -> np.ndarray:
    """The same layer evaluated densely: every routed expert on every token, times a gate that is 0
    for the unselected experts ([TR] §1.1 writes the sum over all mN experts with g = 0 off the top-K)."""
    u = np.asarray(u, dtype=np.float64)
    T = u.shape[0]
    E = len(experts)
    r = route(router_logits(u, w_gate, logit_offset), gate, K, bias, renorm)
    g_full = np.zeros((T, E))
    np.put_along_axis(g_full, r["idx"].astype(np.int64), r["w"], axis=1)
    ffn = (lambda x, p: swiglu_ffn_fp8(x, *p)[0]) if fp8 else (lambda x, p: swiglu_ffn(x, *p))
    h = u + (ffn(u, shared) if shared is not None else 0.0)
    for e in range(E):
        h = h + g_full[:, e:e + 1] * ffn(u, experts[e])
    return h
