"""Plain float64 Mixture-of-Experts FFN layer (oracle side, test infrastructure only).

The pages describe the layer this computes without writing its arithmetic: a
router picks a handful of feed-forward experts per token ("The Billion-Token
Bottleneck", section "The Geometry of the Problem: Why MoE is Different"), and
only those experts' weights take part ("NovaLLM: Running Massive MoE Models
Fully In-Memory", section 2). Readings taken where the pages are silent:

* scores: softmax over the router logits, or an element-wise sigmoid;
* selection key: the logit for softmax routing (monotone in the probability,
  so no exp rounding can create ties); sigmoid(logit) + selection bias for
  sigmoid routing, the bias steering selection only;
* group-limited routing: experts split into n_groups equal consecutive
  groups; a group's score is the sum of its group_topn largest keys; the
  topk_groups best groups are kept (ties to the lower group index), the rest
  are masked before the top-k;
* top-k: keys ordered by (key descending, expert index ascending); output in
  that order;
* gates: renormalised over the selected experts (softmax: the softmax of the
  selected logits; sigmoid: s_j / sum of selected s), then multiplied by
  route_scale;
* grouping: rows ordered expert-major, and within an expert by ascending
  token (a stable counting sort of the flattened (token, slot) list);
* expert: SwiGLU, H = silu(A W_gate) * (A W_up), Y = H W_down, no biases;
* shared expert: always on, added after the routed experts, optionally behind
  a sigmoid scalar gate sigma(x . w_sg);
* combine: out[t] = sum_j gate[t, j] * Y[row of (t, j)] (+ shared term).

Everything is float64 except where a floating-point comparison decides an
integer on the device's own fp32 values (the group score sum in
``select_experts(..., sum_dtype=np.float32)``), which is then taken in fp32 on
both sides.
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np

from . import formats

SOFTMAX, SIGMOID = "softmax", "sigmoid"


# ---------------------------------------------------------------- routing ---

def router_logits(x: np.ndarray, w_r: np.ndarray, logit_bias: np.ndarray | None = None) -> np.ndarray:
    """l = x . W_r (+ logit bias, e.g. a log-prior), float64. x [T, d], W_r [d, E]."""
    logits = np.asarray(x, np.float64) @ np.asarray(w_r, np.float64)
    if logit_bias is not None:
        logits = logits + np.asarray(logit_bias, np.float64)[None, :]
    return logits


def sigmoid(z: np.ndarray) -> np.ndarray:
    z = np.asarray(z, np.float64)
    return 1.0 / (1.0 + np.exp(-z))


def selection_keys(logits: np.ndarray, score_fn: str, select_bias: np.ndarray | None = None) -> np.ndarray:
    """The values top-k ranks experts by: logits (softmax), sigmoid(logits) + bias (sigmoid)."""
    if score_fn == SOFTMAX:
        if select_bias is not None:
            raise ValueError("selection bias is only defined for sigmoid scoring")
        return np.asarray(logits, np.float64)
    if score_fn == SIGMOID:
        s = sigmoid(logits)
        return s if select_bias is None else s + np.asarray(select_bias, np.float64)[None, :]
    raise ValueError(score_fn)


def _order_desc(keys: np.ndarray) -> np.ndarray:
    """Per row, expert indices ordered by key descending, equal keys by ascending index.
    A stable sort of the negated keys keeps equal keys in their original (index) order;
    -0.0 and +0.0 compare equal."""
    return np.argsort(-keys, axis=1, kind="stable")


def group_mask(keys: np.ndarray, n_groups: int, topk_groups: int, group_topn: int,
               sum_dtype=np.float64) -> np.ndarray:
    """Boolean [T, E]: True for experts in the topk_groups best groups. Group g holds
    experts [g*E/n_groups, (g+1)*E/n_groups). Group score = sum of the group's group_topn
    largest keys, added largest first in `sum_dtype`; ties between groups go to the lower
    group index."""
    T, E = keys.shape
    if n_groups <= 1 or topk_groups >= n_groups:
        return np.ones((T, E), dtype=bool)
    if E % n_groups or not (1 <= group_topn <= E // n_groups):
        raise ValueError("bad group configuration")
    gsz = E // n_groups
    kg = np.asarray(keys, sum_dtype).reshape(T, n_groups, gsz)
    top = np.take_along_axis(kg, _order_desc(kg.reshape(T * n_groups, gsz)).reshape(T, n_groups, gsz), axis=2)
    score = top[:, :, 0].copy()
    for i in range(1, group_topn):
        score = (score + top[:, :, i]).astype(sum_dtype)
    keep = _order_desc(score)[:, :topk_groups]
    gmask = np.zeros((T, n_groups), dtype=bool)
    np.put_along_axis(gmask, keep, True, axis=1)
    return np.repeat(gmask, gsz, axis=1)


def select_experts(keys: np.ndarray, k: int, n_groups: int = 1, topk_groups: int = 1,
                   group_topn: int = 0, sum_dtype=np.float64) -> np.ndarray:
    """topk_idx [T, k] int32: the k best experts by (key desc, index asc) among the kept
    groups, best first."""
    keys = np.asarray(keys)
    T, E = keys.shape
    if not (1 <= k <= E):
        raise ValueError("k out of range")
    mask = group_mask(keys, n_groups, topk_groups, group_topn, sum_dtype)
    if k > int(mask[0].sum()):
        raise ValueError("k exceeds the experts left after the group limit")
    masked = np.where(mask, np.asarray(keys, np.float64), -np.inf)
    return _order_desc(masked)[:, :k].astype(np.int32)


def gates(logits: np.ndarray, idx: np.ndarray, score_fn: str, renormalize: bool = True,
          route_scale: float = 1.0) -> np.ndarray:
    """topk_gate [T, k] float64 from the logits of the selected experts."""
    logits = np.asarray(logits, np.float64)
    sel = np.take_along_axis(logits, idx, axis=1)
    if score_fn == SOFTMAX:
        if renormalize:
            z = np.exp(sel - sel.max(axis=1, keepdims=True))
            g = z / z.sum(axis=1, keepdims=True)
        else:
            z = np.exp(logits - logits.max(axis=1, keepdims=True))
            g = np.take_along_axis(z / z.sum(axis=1, keepdims=True), idx, axis=1)
    elif score_fn == SIGMOID:
        s = sigmoid(sel)
        g = s / s.sum(axis=1, keepdims=True) if renormalize else s
    else:
        raise ValueError(score_fn)
    return g * float(route_scale)


@dataclass
class Routing:
    logits: np.ndarray      # [T, E] float64 (including any logit bias)
    keys: np.ndarray        # [T, E] float64 selection keys
    idx: np.ndarray         # [T, k] int32
    gate: np.ndarray        # [T, k] float64
    shared_gate: np.ndarray | None  # [T] float64 or None


def route(x, w_r, *, k, score_fn=SOFTMAX, renormalize=True, route_scale=1.0, n_groups=1,
          topk_groups=1, group_topn=0, logit_bias=None, select_bias=None, w_shared_gate=None) -> Routing:
    """Router scores, group-limited top-k and gates for activations x [T, d] (float64)."""
    logits = router_logits(x, w_r, logit_bias)
    keys = selection_keys(logits, score_fn, select_bias)
    idx = select_experts(keys, k, n_groups, topk_groups, group_topn)
    g = gates(logits, idx, score_fn, renormalize, route_scale)
    sg = None
    if w_shared_gate is not None:
        sg = sigmoid(np.asarray(x, np.float64) @ np.asarray(w_shared_gate, np.float64))
    return Routing(logits, keys, idx, g, sg)


# -------------------------------------------------------------- grouping ---

def expert_counts(idx: np.ndarray, n_experts: int) -> np.ndarray:
    """counts[e] = number of (token, slot) pairs routed to expert e."""
    counts = np.zeros(n_experts, dtype=np.int64)
    np.add.at(counts, np.asarray(idx).ravel(), 1)
    return counts.astype(np.int32)


def expert_offsets(counts: np.ndarray) -> np.ndarray:
    """Exclusive prefix sum, length E+1; offsets[E] = T*k."""
    off = np.zeros(len(counts) + 1, dtype=np.int64)
    running = 0
    for e, c in enumerate(counts):
        off[e] = running
        running += int(c)
    off[-1] = running
    return off.astype(np.int32)


def permutation(idx: np.ndarray, n_experts: int):
    """Stable expert-major grouping of the flattened pairs p = t*k + j.
    Returns (offsets [E+1], perm_src [T*k]: row -> p, perm_dst [T*k]: p -> row)."""
    flat = np.asarray(idx).ravel()
    offsets = expert_offsets(expert_counts(idx, n_experts))
    cursor = offsets[:-1].astype(np.int64).copy()
    perm_src = np.empty(flat.size, dtype=np.int32)
    for p, e in enumerate(flat.tolist()):       # ascending p = ascending token
        perm_src[cursor[e]] = p
        cursor[e] += 1
    perm_dst = np.empty_like(perm_src)
    perm_dst[perm_src] = np.arange(flat.size, dtype=np.int32)
    return offsets, perm_src, perm_dst


# ------------------------------------------------------------ expert FFN ---

def silu(z: np.ndarray) -> np.ndarray:
    return z * sigmoid(z)


def quantize_activations(a: np.ndarray, mode) -> np.ndarray:
    """The expert inputs as the GEMMs see them (float64): unchanged for mode False/None;
    True or "e4m3": the per-row per-128 e4m3 quantisation with fp32 scales (the fp8
    workload); "mxfp8": the OCP MXFP8 conversion (E4M3 with one power-of-two scale per 32), the
    activations of MXFP4 experts on the block-scaled matrix instructions."""
    if not mode:
        return np.asarray(a, np.float64)
    if mode is True or mode == "e4m3":
        q, s = formats.quantize_rows_e4m3(a)
        return formats.dequantize_rows(q, s)
    if mode == "mxfp8":
        q, e = formats.quantize_rows_mxfp8(a)
        return formats.dequantize_rows_mxfp8(q, e)
    raise ValueError(f"quantize_activations: unknown mode {mode!r}")


def swiglu_ffn(a: np.ndarray, w_gate: np.ndarray, w_up: np.ndarray, w_down: np.ndarray,
               quant_hidden=False) -> np.ndarray:
    """Y = (silu(A W_gate) * (A W_up)) W_down in float64. A [n, d], W_gate/W_up [d, F],
    W_down [F, d]. With quant_hidden (a quantize_activations mode) the hidden activations
    go through the same quantisation as the inputs before the down projection."""
    a = np.asarray(a, np.float64)
    h = silu(a @ w_gate) * (a @ w_up)
    return quantize_activations(h, quant_hidden) @ w_down


# ---------------------------------------------------------------- layer ---

@dataclass
class ExpertWeights:
    """One expert's weights as float64 [d, F], [d, F], [F, d]."""
    w_gate: np.ndarray
    w_up: np.ndarray
    w_down: np.ndarray


def combine(gate: np.ndarray, y_rows: np.ndarray, perm_dst: np.ndarray, shared_y=None,
            shared_gate=None) -> np.ndarray:
    """out[t] = sum_j gate[t, j] * Y[perm_dst[t*k + j]] (+ shared_gate[t] * S[t])."""
    T, k = gate.shape
    out = np.zeros((T, y_rows.shape[1]), dtype=np.float64)
    for j in range(k):
        rows = perm_dst.reshape(T, k)[:, j]
        out += gate[:, j:j + 1] * y_rows[rows]
    if shared_y is not None:
        sg = np.ones(T) if shared_gate is None else np.asarray(shared_gate, np.float64)
        out += sg[:, None] * shared_y
    return out


def moe_layer(x: np.ndarray, routing: Routing, expert, n_experts: int, *, shared=None,
              quant_act=False, tokens=None) -> np.ndarray:
    """Layer output [T', d] float64 for the tokens in `tokens` (all when None).

    `expert(e)` returns an ExpertWeights (float64). `shared` is an ExpertWeights or None.
    With quant_act (a quantize_activations mode: True/"e4m3" for the fp8 workload, "mxfp8"
    for MXFP4 experts on the block-scaled matrix instructions) the expert inputs (x, and the
    hidden activations) go through that quantisation. The routed part follows the
    grouped formulation: rows grouped by expert (stable), each expert run once on its
    rows, then the gate-weighted combine back to token order."""
    x = np.asarray(x, np.float64)
    T = x.shape[0]
    tokens = np.arange(T) if tokens is None else np.asarray(tokens)
    idx = routing.idx[tokens]
    k = idx.shape[1]
    xa = x[tokens]
    xa = quantize_activations(xa, quant_act)
    offsets, perm_src, perm_dst = permutation(idx, n_experts)
    y_rows = np.zeros((idx.size, x.shape[1]), dtype=np.float64)
    for e in range(n_experts):
        lo, hi = int(offsets[e]), int(offsets[e + 1])
        if hi == lo:
            continue
        w = expert(e)
        a = xa[perm_src[lo:hi] // k]
        y_rows[lo:hi] = swiglu_ffn(a, w.w_gate, w.w_up, w.w_down, quant_hidden=quant_act)
    shared_y = None
    if shared is not None:
        shared_y = swiglu_ffn(xa, shared.w_gate, shared.w_up, shared.w_down, quant_hidden=quant_act)
    sg = None if routing.shared_gate is None else routing.shared_gate[tokens]
    return combine(routing.gate[tokens], y_rows, perm_dst, shared_y, sg)
