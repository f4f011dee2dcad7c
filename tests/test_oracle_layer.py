"""Pins for the oracle's grouping, expert FFN and layer: library routines (numpy
bincount / cumsum / stable argsort, torch fp64 matmul and silu), invariants,
the dense-FFN identity and a permutation-free brute-force layer."""
import numpy as np
import pytest
import torch

from oracle import formats, moe


def test_counts_offsets_permutation_invariants():
    rng = np.random.default_rng(1)
    for T, E, k in [(1, 4, 1), (17, 8, 2), (64, 60, 4), (300, 256, 8), (5, 3, 3)]:
        keys = rng.standard_normal((T, E))
        idx = moe.select_experts(keys, k)
        counts = moe.expert_counts(idx, E)
        assert counts.sum() == T * k
        assert np.array_equal(counts, np.bincount(idx.ravel(), minlength=E))
        off, src, dst = moe.permutation(idx, E)
        assert off[0] == 0 and off[-1] == T * k
        assert np.array_equal(off[1:], np.cumsum(counts))
        assert np.array_equal(np.sort(src), np.arange(T * k))           # bijection
        assert np.array_equal(dst[src], np.arange(T * k))               # inverse
        assert np.array_equal(src, np.argsort(idx.ravel(), kind="stable"))
        flat = idx.ravel()
        for e in range(E):
            seg = src[off[e]:off[e + 1]]
            assert np.all(flat[seg] == e)
            assert np.all(np.diff(seg // k) > 0)                        # tokens ascending


def test_silu_closed_forms():
    assert moe.silu(np.array([0.0]))[0] == 0.0
    np.testing.assert_allclose(moe.silu(np.array([40.0])), [40.0], rtol=1e-15)
    assert abs(moe.silu(np.array([-40.0]))[0]) < 1e-15
    np.testing.assert_allclose(moe.silu(np.array([1.0])), [1.0 / (1.0 + np.exp(-1.0))], rtol=1e-15)


def test_swiglu_matches_torch():
    rng = np.random.default_rng(2)
    a = rng.standard_normal((9, 32))
    wg, wu = rng.standard_normal((32, 48)), rng.standard_normal((32, 48))
    wd = rng.standard_normal((48, 32))
    ta = torch.from_numpy(a)
    ref = (torch.nn.functional.silu(ta @ torch.from_numpy(wg)) * (ta @ torch.from_numpy(wu))) @ torch.from_numpy(wd)
    np.testing.assert_allclose(moe.swiglu_ffn(a, wg, wu, wd), ref.numpy(), rtol=1e-12, atol=1e-12)


def _rand_layer(rng, T, d, E, F, identical=False):
    x = rng.standard_normal((T, d))
    w_r = rng.standard_normal((d, E)) / np.sqrt(d)
    base = moe.ExpertWeights(rng.standard_normal((d, F)) / np.sqrt(d), rng.standard_normal((d, F)) / np.sqrt(d),
                             rng.standard_normal((F, d)) / np.sqrt(F))
    ws = [base if identical else moe.ExpertWeights(rng.standard_normal((d, F)) / np.sqrt(d),
                                                  rng.standard_normal((d, F)) / np.sqrt(d),
                                                  rng.standard_normal((F, d)) / np.sqrt(F)) for _ in range(E)]
    return x, w_r, ws


def _brute_layer(x, r, ws, shared=None):
    """Permutation-free token-major loop: out[t] = sum_{e in sel(t)} g * FFN_e(x_t) (+ shared)."""
    out = np.zeros_like(x)
    for t in range(x.shape[0]):
        for j, e in enumerate(r.idx[t]):
            w = ws[e]
            out[t] += r.gate[t, j] * moe.swiglu_ffn(x[t:t + 1], w.w_gate, w.w_up, w.w_down)[0]
        if shared is not None:
            sg = 1.0 if r.shared_gate is None else r.shared_gate[t]
            out[t] += sg * moe.swiglu_ffn(x[t:t + 1], shared.w_gate, shared.w_up, shared.w_down)[0]
    return out


@pytest.mark.parametrize("score_fn,k,groups", [("softmax", 2, (1, 1, 0)), ("softmax", 3, (1, 1, 0)),
                                               ("sigmoid", 4, (4, 2, 2))])
def test_layer_equals_brute_force(score_fn, k, groups):
    rng = np.random.default_rng(3)
    x, w_r, ws = _rand_layer(rng, 13, 16, 8, 24)
    bias = rng.standard_normal(8) * 0.1 if score_fn == "sigmoid" else None
    r = moe.route(x, w_r, k=k, score_fn=score_fn, route_scale=2.5 if score_fn == "sigmoid" else 1.0,
                  n_groups=groups[0], topk_groups=groups[1], group_topn=groups[2], select_bias=bias)
    got = moe.moe_layer(x, r, lambda e: ws[e], 8)
    np.testing.assert_allclose(got, _brute_layer(x, r, ws), rtol=1e-12, atol=1e-12)
    sub = np.array([0, 5, 12])
    np.testing.assert_allclose(moe.moe_layer(x, r, lambda e: ws[e], 8, tokens=sub), got[sub], rtol=1e-12, atol=1e-12)


def test_layer_with_gated_shared_expert_equals_brute_force():
    rng = np.random.default_rng(4)
    x, w_r, ws = _rand_layer(rng, 11, 16, 6, 20)
    shared = moe.ExpertWeights(rng.standard_normal((16, 40)), rng.standard_normal((16, 40)), rng.standard_normal((40, 16)))
    wsg = rng.standard_normal(16)
    r = moe.route(x, w_r, k=2, w_shared_gate=wsg)
    got = moe.moe_layer(x, r, lambda e: ws[e], 6, shared=shared)
    np.testing.assert_allclose(got, _brute_layer(x, r, ws, shared), rtol=1e-12, atol=1e-12)


def test_dense_identity_softmax():
    """top_k = E over identical experts with renormalised gates reproduces the dense FFN."""
    rng = np.random.default_rng(5)
    x, w_r, ws = _rand_layer(rng, 10, 16, 5, 24, identical=True)
    r = moe.route(x, w_r, k=5)
    w = ws[0]
    np.testing.assert_allclose(moe.moe_layer(x, r, lambda e: ws[e], 5),
                               moe.swiglu_ffn(x, w.w_gate, w.w_up, w.w_down), rtol=1e-12, atol=1e-12)


def test_dense_identity_sigmoid_grouped_scaled():
    """Same identity for sigmoid routing with all groups kept: 2.5 x the dense FFN."""
    rng = np.random.default_rng(6)
    x, w_r, ws = _rand_layer(rng, 10, 16, 8, 24, identical=True)
    r = moe.route(x, w_r, k=8, score_fn="sigmoid", route_scale=2.5, n_groups=4, topk_groups=4,
                  group_topn=2, select_bias=rng.standard_normal(8) * 0.1)
    w = ws[0]
    np.testing.assert_allclose(moe.moe_layer(x, r, lambda e: ws[e], 8),
                               2.5 * moe.swiglu_ffn(x, w.w_gate, w.w_up, w.w_down), rtol=1e-12, atol=1e-12)


def test_single_expert_is_ffn():
    rng = np.random.default_rng(7)
    x, w_r, ws = _rand_layer(rng, 6, 16, 1, 8)
    r = moe.route(x, w_r, k=1)
    assert np.all(r.gate == 1.0)
    w = ws[0]
    np.testing.assert_allclose(moe.moe_layer(x, r, lambda e: ws[e], 1),
                               moe.swiglu_ffn(x, w.w_gate, w.w_up, w.w_down), rtol=1e-13)


def test_quantised_layer_matches_explicit_dequantisation():
    """The fp8 path: layer with quant_act equals running the brute-force loop on the
    dequantised activations, with the hidden layer quantised per row (torch fp8 cast)."""
    rng = np.random.default_rng(8)
    x, w_r, ws = _rand_layer(rng, 7, 128, 4, 128)
    r = moe.route(x, w_r, k=2)
    got = moe.moe_layer(x, r, lambda e: ws[e], 4, quant_act=True)

    def tq(a):  # per-row per-128 quantise/dequantise via torch's e4m3 cast
        t = torch.from_numpy(a.astype(np.float32)).view(a.shape[0], -1, 128)
        s = t.abs().amax(dim=2, keepdim=True) / 448.0
        q = (t / s).clamp(-448, 448).to(torch.float8_e4m3fn).to(torch.float64)
        return (q * s.double()).view(a.shape).numpy()

    xq = tq(x)
    ref = np.zeros_like(x)
    for t in range(7):
        for j, e in enumerate(r.idx[t]):
            w = ws[e]
            h = moe.silu(xq[t:t + 1] @ w.w_gate) * (xq[t:t + 1] @ w.w_up)
            ref[t] += r.gate[t, j] * (tq(h) @ w.w_down)[0]
    np.testing.assert_allclose(got, ref, rtol=1e-12, atol=1e-12)


def test_mxfp8_layer_matches_explicit_dequantisation():
    """The MXFP4-prefill activations: the layer with quant_act="mxfp8" equals the brute-force
    token loop on inputs and hidden activations quantised per 32 with a power-of-two scale,
    written here with torch's e4m3 cast and the shared exponent from the float's exponent
    field (frexp)."""
    rng = np.random.default_rng(9)
    x, w_r, ws = _rand_layer(rng, 6, 64, 4, 96)
    r = moe.route(x, w_r, k=2)
    got = moe.moe_layer(x, r, lambda e: ws[e], 4, quant_act="mxfp8")

    def tq(a):
        b = a.reshape(a.shape[0], -1, 32)
        _, ex = np.frexp(np.abs(b).max(axis=2, keepdims=True))
        s = np.ldexp(1.0, ex - 1 - 8)
        q = torch.from_numpy(np.clip(b / s, -448, 448)).to(torch.float8_e4m3fn).to(torch.float64).numpy()
        return (q * s).reshape(a.shape)

    xq = tq(x)
    ref = np.zeros_like(x)
    for t in range(6):
        for j, e in enumerate(r.idx[t]):
            w = ws[e]
            h = moe.silu(xq[t:t + 1] @ w.w_gate) * (xq[t:t + 1] @ w.w_up)
            ref[t] += r.gate[t, j] * (tq(h) @ w.w_down)[0]
    np.testing.assert_allclose(got, ref, rtol=1e-12, atol=1e-12)
