"""The sparse-MoE layer forward, written out step by step in fp64.
TEST INFRASTRUCTURE ONLY (see the package docstring).

Sources (page titles abbreviated; sections as the pages number or name them):

* [Qwen3] "Qwen3-MoE low-latency inference on Atlas A3 / 950 clusters"
  page: "MoE TP optimisation -> compute decomposition" (expert FFN
  x = down(SiLU(gate(x)) * up(x)); gate_proj and up_proj concatenated into
  w13; npu_swiglu splits the last dimension in two and returns
  SiLU(first half) * second half) and "GMM enablement and routing
  optimisation" (gating top-k softmax fused, init_routing gives the experts'
  sort order, compute_expert_tokens gives tokens per expert, grouped matmul
  computes all experts, finalize_routing re-orders expert outputs back to
  tokens and takes the weighted sum); "fused RMSNorm + Cast" (the gate input
  is fp32).
* [Hy3] "Hy3 295B MoE on Atlas A3" page: section 1.1 (one shared expert per
  MoE layer, gate/up 4096->1536, down 1536->4096), section 1.3 (sigmoid
  router; learnable e_score_correction_bias takes part in routing scores;
  top-k weights x 2.826; the router call with k, bias, sigmoid norm type,
  routed_scaling_factor and eps 1e-20), section 5.1 (the model adds the bias
  after the sigmoid and it only affects top-k selection).

Readings where the pages are silent (each also listed in the design notes):

* softmax gating: the k largest logits are selected and the softmax is taken
  over the selected ones.  Softmax-then-top-k-then-renormalise gives the same
  weights because the full denominator cancels; selecting on raw logits avoids
  ties created by rounding probabilities.
* ties between equal keys go to the lower expert id; a token's k slots are
  ordered by key descending, then id ascending.
* sigmoid gating: s = sigmoid(logit) in fp64, key = s + bias (fp64) decides
  selection only; weight_j = s_j / (sum of selected s + eps) * routed_scale.
* the routing permutation is the stable sort of pairs p = t*k + j by expert.
* the SwiGLU output is rounded to bf16 (it is the bf16 input of the down
  projection); the final output is rounded to bf16; everything else fp64.
* the shared expert is added with weight 1 (not scaled by 2.826).
"""
from __future__ import annotations

from typing import Callable, Optional, Sequence, Tuple

import numpy as np

from . import mx

F64 = np.float64


# ----------------------------------------------------------------- S1 ------

def router_logits(x, wr) -> np.ndarray:
    """L[t, e] = sum_h x[t, h] * Wr[e, h], accumulated in fp64 and rounded to
    fp32 (the gate runs in fp32: [Qwen3] "fused RMSNorm + Cast").
    x: [T, H] (bf16 values), wr: [E, H] fp32."""
    x = np.asarray(x, dtype=F64)
    wr = np.asarray(wr, dtype=F64)
    return (x @ wr.T).astype(np.float32)


# ----------------------------------------------------------------- S2 ------

def _select_topk(key: np.ndarray, k: int) -> np.ndarray:
    """Per row, the k column ids with the largest key; ties -> lower id.
    Rows are ordered by (key descending, id ascending)."""
    T, E = key.shape
    ids = np.broadcast_to(np.arange(E), (T, E))
    order = np.lexsort((ids, -key), axis=-1)  # primary: -key, secondary: id
    return order[:, :k]


def gate_topk_softmax(logits, k: int, bias=None) -> Tuple[np.ndarray, np.ndarray]:
    """[Qwen3] fused gating top-k softmax.  key = fl32(L + b) (b optional
    router bias, added to the logits), top-k on key, weights = softmax over
    the selected keys (fp64, rounded to fp32).  Returns ids int32 [T,k],
    weights fp32 [T,k]."""
    L = np.asarray(logits, dtype=np.float32)
    key32 = L if bias is None else (L + np.asarray(bias, dtype=np.float32)[None, :])
    key = key32.astype(F64)
    ids = _select_topk(key, k)
    sel = np.take_along_axis(key, ids, axis=1)
    z = np.exp(sel - sel[:, :1])
    w = z / z.sum(axis=1, keepdims=True)
    return ids.astype(np.int32), w.astype(np.float32)


def gate_topk_sigmoid(logits, k: int, bias=None, routed_scale: float = 1.0,
                      eps: float = 1e-20) -> Tuple[np.ndarray, np.ndarray]:
    """[Hy3] sections 1.3 and 5.1: s = sigmoid(L); key = s + bias decides the
    top-k only; weights are the unbiased s of the selected experts divided by
    (their sum + eps) and multiplied by routed_scale."""
    L = np.asarray(logits, dtype=np.float32).astype(F64)
    s = 1.0 / (1.0 + np.exp(-L))
    key = s if bias is None else s + np.asarray(bias, dtype=np.float32).astype(F64)[None, :]
    ids = _select_topk(key, k)
    ssel = np.take_along_axis(s, ids, axis=1)
    scale = F64(np.float32(routed_scale))
    w = ssel / (ssel.sum(axis=1, keepdims=True) + F64(eps)) * scale
    return ids.astype(np.int32), w.astype(np.float32)


# -------------------------------------------------------------- S3, S4 -----

def route(topk_ids, E: int):
    """[Qwen3] init_routing + compute_expert_tokens.

    counts[e]   = number of pairs routed to expert e (tokens per expert)
    offsets     = exclusive prefix sum of counts, length E+1
    sorted_pair = pairs p = t*k + j ordered by expert, ascending p inside an
                  expert (a stable sort by expert id)
    pair_pos    = inverse permutation: pair_pos[sorted_pair[r]] = r
    """
    flat = np.asarray(topk_ids, dtype=np.int64).reshape(-1)
    counts = np.array([int(np.count_nonzero(flat == e)) for e in range(E)], dtype=np.int64)
    offsets = np.zeros(E + 1, dtype=np.int64)
    offsets[1:] = np.cumsum(counts)
    segs = [np.nonzero(flat == e)[0] for e in range(E)]
    sorted_pair = np.concatenate(segs) if segs else np.zeros(0, np.int64)
    pair_pos = np.empty_like(sorted_pair)
    pair_pos[sorted_pair] = np.arange(sorted_pair.size)
    return (counts.astype(np.int32), offsets.astype(np.int32),
            sorted_pair.astype(np.int32), pair_pos.astype(np.int32))


# -------------------------------------------------------------- S5, S6 -----

def silu(g):
    g = np.asarray(g, dtype=F64)
    with np.errstate(over="ignore"):
        return g / (1.0 + np.exp(-g))


def expert_ffn(xrows, w13, w2, act: str = "bf16", act_exponents=None,
               stats: Optional[dict] = None) -> np.ndarray:
    """[Qwen3] expert FFN x -> down(SiLU(gate x) * up x) with w13 = gate_proj
    rows followed by up_proj rows (weights in [out, in] layout).

    act = "bf16": the SwiGLU output is rounded to bf16 before the down
    projection; act = "mxfp8": it is quantised to MXFP8 along the
    intermediate dimension and dequantised ([Hy3] section 5.2: SwiGLU with
    group quantisation).  act_exponents ([m, I/32], mxfp8 only): block
    exponents decided elsewhere, used instead of the rule's own (see
    mx.mxfp8_quantize).  If ``stats`` is given, the exact block maxima of
    the SwiGLU output are stored in stats["amax"] ([m, I/32]).
    Returns y [m, H] fp64."""
    xrows = np.asarray(xrows, dtype=F64)
    w13 = np.asarray(w13, dtype=F64)
    w2 = np.asarray(w2, dtype=F64)
    I = w13.shape[0] // 2
    g = xrows @ w13[:I].T
    u = xrows @ w13[I:].T
    a = silu(g) * u
    if stats is not None and act == "mxfp8":
        stats["amax"] = np.abs(a).reshape(a.shape[0], I // 32, 32).max(-1)
    if act == "bf16":
        a = mx.bf16_round(a)
    elif act == "mxfp8":
        a = mx.mxfp8_dequant(*mx.mxfp8_quantize(a, act_exponents))
    else:
        raise ValueError(act)
    return a @ w2.T


# ----------------------------------------------------------------- S7 ------

def combine(y_rows, pair_pos, topk_w, shared=None) -> np.ndarray:
    """[Qwen3] finalize_routing: out[t] = sum_j w[t,j] * y[pair_pos[t*k+j]]
    (+ shared[t], [Hy3] section 1.1), in fp64, rounded to bf16."""
    w = np.asarray(topk_w, dtype=np.float32).astype(F64)
    T, k = w.shape
    y_rows = np.asarray(y_rows, dtype=F64)
    pos = np.asarray(pair_pos).reshape(T, k)
    out = np.zeros((T, y_rows.shape[1]), dtype=F64)
    for j in range(k):
        out += w[:, j:j + 1] * y_rows[pos[:, j]]
    if shared is not None:
        out += np.asarray(shared, dtype=F64)
    return mx.bf16_round(out)


# --------------------------------------------------------------- layer -----

def gate(logits, k: int, mode: str, bias=None, routed_scale: float = 1.0, eps: float = 1e-20):
    if mode == "softmax":
        return gate_topk_softmax(logits, k, bias)
    if mode == "sigmoid":
        return gate_topk_sigmoid(logits, k, bias, routed_scale, eps)
    raise ValueError(mode)


def layer_forward(x, wr, k: int, mode: str, expert_weights: Callable[[int], tuple],
                  E: int, bias=None, routed_scale: float = 1.0, eps: float = 1e-20,
                  shared_weights: Optional[tuple] = None, fmt: str = "bf16",
                  logits=None, tokens: Optional[Sequence[int]] = None,
                  act_exponents=None, shared_act_exponents=None) -> dict:
    """The whole layer: S1 logits, S2 gate, S3/S4 routing, S5/S6 expert FFNs
    over the permuted rows, S7 combine (+ shared expert).

    expert_weights(e) returns the expert's (w13 [2I,H], w2 [H,I]) as values
    (already decoded for MX weights).  fmt "w4a8" quantises x to MXFP8 before
    the experts and the SwiGLU output to MXFP8 before the down projection;
    the router stays on the unquantised x.  If ``logits`` is given it is used
    for gating instead of recomputing them (the GPU's fp32 logits, so that
    selection is decided on identical keys).  If ``tokens`` is given, the
    expert FFNs and the combine are evaluated only for those tokens (routing
    is still computed for all tokens); ``out`` then has one row per listed
    token.

    act_exponents ([T*k, I/32], indexed by permuted row) and
    shared_act_exponents ([T, I_s/32], by token), W4A8 only: the MXFP8 block
    exponents of the SwiGLU outputs decided by another computation (the
    GPU's, from its own fp32 values), used instead of the rule's own, like
    ``logits`` for the selection.  The exact block maxima of the SwiGLU
    outputs are returned (act_amax [T*k, I/32] by permuted row, NaN for rows
    not evaluated; shared_act_amax [len(tokens), I_s/32]) so that a caller
    can check that the exponents it passed differ from the rule's only
    where the rule's own decision sits at a power of two.
    """
    x = np.asarray(x, dtype=F64)
    T = x.shape[0]
    L_ref = router_logits(x, wr)
    L = L_ref if logits is None else np.asarray(logits, dtype=np.float32)
    ids, w = gate(L, k, mode, bias, routed_scale, eps)
    counts, offsets, sorted_pair, pair_pos = route(ids, E)
    if fmt == "w4a8":
        xin = mx.mxfp8_dequant(*mx.mxfp8_quantize(x))
        act = "mxfp8"
    else:
        xin = x
        act = "bf16"
    toks = np.arange(T) if tokens is None else np.asarray(tokens, dtype=np.int64)
    want = np.zeros(T, dtype=bool)
    want[toks] = True
    H = x.shape[1]
    R = T * k
    y = np.zeros((R, H), dtype=F64) if tokens is None else {}
    act_amax = None
    for e in range(E):
        rows = np.arange(offsets[e], offsets[e + 1])
        if rows.size == 0:
            continue
        t_of_row = sorted_pair[rows] // k
        keep = want[t_of_row]
        if not keep.any():
            continue
        w13, w2 = expert_weights(e)
        st = {}
        ex = None if act_exponents is None else np.asarray(act_exponents)[rows[keep]]
        ye = expert_ffn(xin[t_of_row[keep]], w13, w2, act, ex, st)
        if "amax" in st:
            if act_amax is None:
                act_amax = np.full((R, st["amax"].shape[1]), np.nan)
            act_amax[rows[keep]] = st["amax"]
        if tokens is None:
            y[rows[keep]] = ye
        else:
            for r, v in zip(rows[keep], ye):
                y[int(r)] = v
    shared = None
    shared_amax = None
    if shared_weights is not None:
        st = {}
        ex = None if shared_act_exponents is None else np.asarray(shared_act_exponents)[toks]
        shared = expert_ffn(xin[toks], shared_weights[0], shared_weights[1], act, ex, st)
        shared_amax = st.get("amax")
    if tokens is None:
        out = combine(y, pair_pos, w, shared)
    else:
        pos = pair_pos.reshape(T, k)[toks]
        yrows = np.stack([y[int(r)] for r in pos.reshape(-1)]) if toks.size else np.zeros((0, H))
        out = combine(yrows, np.arange(pos.size), w[toks], shared)
    return dict(logits=L_ref, ids=ids, w=w, counts=counts, offsets=offsets,
                sorted_pair=sorted_pair, pair_pos=pair_pos, out=out,
                x_used=xin if fmt == "w4a8" else None,
                act_amax=act_amax, shared_act_amax=shared_amax)
