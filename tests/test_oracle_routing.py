"""Pins for the oracle's router: brute force over expert and group subsets,
closed forms, invariants and library routines (numpy lexsort, scipy softmax)."""
import itertools
import os

import numpy as np
import pytest
from scipy.special import expit, softmax

from oracle import moe

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _beats(ka, a, kb, b):
    return ka > kb or (ka == kb and a < b)


def _brute_topk(keys_row, k, allowed=None):
    E = len(keys_row)
    allowed = range(E) if allowed is None else allowed
    valid = []
    for S in itertools.combinations(allowed, k):
        rest = [j for j in allowed if j not in S]
        if all(_beats(keys_row[i], i, keys_row[j], j) for i in S for j in rest):
            valid.append(S)
    assert len(valid) == 1
    S = list(valid[0])
    # best first: sort by the same total order, via pairwise comparison counts
    return sorted(S, key=lambda i: sum(_beats(keys_row[j], j, keys_row[i], i) for j in S))


@pytest.mark.parametrize("E,k", [(4, 1), (4, 2), (6, 3), (8, 2), (8, 3)])
def test_topk_brute_force(E, k):
    rng = np.random.default_rng(E * 10 + k)
    for trial in range(60):
        if trial % 2:
            keys = rng.integers(-2, 3, (1, E)).astype(np.float64)    # many ties
        else:
            keys = rng.standard_normal((1, E))
        got = moe.select_experts(keys, k)[0].tolist()
        assert got == _brute_topk(keys[0], k)


def test_topk_matches_lexsort():
    rng = np.random.default_rng(3)
    keys = rng.integers(-3, 4, (200, 16)).astype(np.float64)
    got = moe.select_experts(keys, 5)
    for t in range(200):
        order = np.lexsort((np.arange(16), -keys[t]))
        assert got[t].tolist() == order[:5].tolist()


def test_top1_is_argmax_first_index():
    rng = np.random.default_rng(4)
    keys = rng.integers(0, 3, (300, 7)).astype(np.float64)
    assert np.array_equal(moe.select_experts(keys, 1)[:, 0], np.argmax(keys, axis=1))


def test_signed_zero_ties():
    keys = np.array([[-0.0, 0.0, -1.0]])
    assert moe.select_experts(keys, 2)[0].tolist() == [0, 1]


def _brute_group_topk(keys_row, k, n_groups, topk_groups, topn):
    E = len(keys_row)
    g = E // n_groups
    gscore = []
    for gi in range(n_groups):
        vals = sorted(keys_row[gi * g:(gi + 1) * g], reverse=True)[:topn]
        gscore.append(sum(vals))
    kept = _brute_topk(np.array(gscore), topk_groups)
    allowed = [e for e in range(E) if e // g in kept]
    return _brute_topk(keys_row, k, allowed)


@pytest.mark.parametrize("E,G,TG,N,k", [(16, 8, 4, 2, 4), (16, 8, 4, 1, 3), (24, 8, 3, 2, 5), (8, 4, 2, 2, 3)])
def test_group_limited_brute_force(E, G, TG, N, k):
    rng = np.random.default_rng(E + G + TG + N + k)
    for trial in range(40):
        if trial % 2:
            keys = rng.integers(0, 4, (1, E)).astype(np.float64)
        else:
            keys = rng.standard_normal((1, E))
        got = moe.select_experts(keys, k, G, TG, N)[0].tolist()
        assert got == _brute_group_topk(keys[0], k, G, TG, N)


def test_group_limit_all_groups_reduces_to_plain():
    rng = np.random.default_rng(5)
    keys = rng.standard_normal((50, 32))
    assert np.array_equal(moe.select_experts(keys, 6, 8, 8, 2), moe.select_experts(keys, 6))
    assert np.array_equal(moe.select_experts(keys, 6, 1, 1, 2), moe.select_experts(keys, 6))


def test_group_sum_fp32_mode():
    # group 1 = {1.0, 2^-24}: its fp64 sum beats group 0 = {1.0, 0.0}, but in fp32
    # 1 + 2^-24 rounds (to even) back to 1.0, the groups tie and the lower group wins.
    eps = 2.0 ** -24
    keys = np.array([[1.0, 0.0, 1.0, eps]])
    assert moe.select_experts(keys, 1, 2, 1, 2, np.float64)[0, 0] == 2
    assert moe.select_experts(keys.astype(np.float32), 1, 2, 1, 2, np.float32)[0, 0] == 0


def test_softmax_gates_renormalised():
    rng = np.random.default_rng(6)
    logits = rng.standard_normal((100, 12)) * 3
    idx = moe.select_experts(logits, 4)
    g = moe.gates(logits, idx, "softmax")
    np.testing.assert_allclose(g.sum(axis=1), 1.0, rtol=0, atol=1e-12)
    sel = np.take_along_axis(logits, idx, axis=1)
    np.testing.assert_allclose(g, softmax(sel, axis=1), rtol=1e-13, atol=0)
    full = softmax(logits, axis=1)
    ref = np.take_along_axis(full, idx, axis=1)
    np.testing.assert_allclose(g, ref / ref.sum(axis=1, keepdims=True), rtol=1e-12)
    g_raw = moe.gates(logits, idx, "softmax", renormalize=False)
    np.testing.assert_allclose(g_raw, ref, rtol=1e-12)
    # shift invariance of selection and gates
    shifted = logits + 17.0
    assert np.array_equal(moe.select_experts(shifted, 4), idx)
    np.testing.assert_allclose(moe.gates(shifted, idx, "softmax"), g, rtol=1e-12)


def test_sigmoid_gates_scaled():
    rng = np.random.default_rng(7)
    logits = rng.standard_normal((100, 32))
    bias = rng.standard_normal(32) * 0.1
    keys = moe.selection_keys(logits, "sigmoid", bias)
    np.testing.assert_allclose(keys, expit(logits) + bias, rtol=1e-15)
    idx = moe.select_experts(keys, 8, 8, 4, 2)
    g = moe.gates(logits, idx, "sigmoid", route_scale=2.5)
    np.testing.assert_allclose(g.sum(axis=1), 2.5, atol=1e-12)
    s = np.take_along_axis(expit(logits), idx, axis=1)
    np.testing.assert_allclose(g, 2.5 * s / s.sum(axis=1, keepdims=True), rtol=1e-13)
    # without bias, sigmoid top-k equals top-k on the logits (sigmoid is monotone)
    assert np.array_equal(moe.select_experts(moe.selection_keys(logits, "sigmoid"), 8),
                          moe.select_experts(logits, 8))


def test_route_closed_forms():
    cases = {}
    for line in open(os.path.join(GOLDEN, "route_closed_form.txt")):
        line = line.split("#")[0].strip()
        if line:
            parts = line.split()
            i, gi = parts.index("idx"), parts.index("gate")
            cases[parts[0]] = ([int(v) for v in parts[i + 1:gi]], [float(v) for v in parts[gi + 1:]])
    r = moe.route(np.ones((1, 4)), np.diag(np.log([1.0, 2.0, 3.0, 4.0])), k=2)
    assert r.idx[0].tolist() == cases["softmax_top2"][0]
    np.testing.assert_allclose(r.gate[0], cases["softmax_top2"][1], rtol=1e-14)
    r = moe.route(np.ones((1, 4)), np.zeros((4, 4)), k=2, score_fn="sigmoid", route_scale=2.5)
    assert r.idx[0].tolist() == cases["sigmoid_tie_top2_scaled"][0]
    np.testing.assert_allclose(r.gate[0], cases["sigmoid_tie_top2_scaled"][1], rtol=1e-14)
    r = moe.route(np.ones((1, 3)), np.zeros((3, 3)), k=1, score_fn="sigmoid",
                  select_bias=np.array([0.0, 0.1, -0.1]))
    assert r.idx[0].tolist() == cases["sigmoid_bias_top1"][0]
    np.testing.assert_allclose(r.gate[0], cases["sigmoid_bias_top1"][1], rtol=1e-14)


def test_logit_bias_and_shared_gate():
    rng = np.random.default_rng(8)
    x = rng.standard_normal((10, 6))
    w = rng.standard_normal((6, 5))
    b = rng.standard_normal(5)
    wsg = rng.standard_normal(6)
    r = moe.route(x, w, k=2, logit_bias=b, w_shared_gate=wsg)
    np.testing.assert_allclose(r.logits, x @ w + b, rtol=1e-14)
    np.testing.assert_allclose(r.shared_gate, expit(x @ wsg), rtol=1e-14)
