"""The fused decode step (moe_decode_step) through the C ABI: routing beside the shared expert's
gate/up, the shared down beside the routed gate/up, then the routed down with the combine.

Its contract is bit-identity with the separate calls (moe_route_permute, then the batched FFN
and the combine), so each case runs the same layer both ways and compares every output bit for
bit; the separate calls are themselves checked against the float64 oracle elsewhere, and here
the step's own output is also compared with the oracle and its indices with the oracle's
selection on the device's keys."""
import numpy as np
import pytest
import torch

from expert_offloaded_ffn_amd import binding as B
from expert_offloaded_ffn_amd import synth
from expert_offloaded_ffn_amd.layer import MoELayer
from oracle import moe
from parity_util import (assert_close, check_exact_indices, decode, oracle_expert, oracle_route, route_agreement, say,
                         to_np)

pytestmark = pytest.mark.gpu
DEV = "cuda"
ROUTE_KEYS = ("scores", "idx", "gate", "counts", "offsets", "perm_src", "perm_dst")


def _x(cfg, xi, T):
    xs = synth.gen_x(cfg, xi, T=T)
    return xs, torch.from_numpy(xs.view(np.int16)).view(torch.bfloat16).to(DEV)


def _layers(cfg, with_shared):
    w = dict(router=synth.gen_router(cfg), experts=synth.gen_experts(cfg))
    kw = {}
    if with_shared and cfg.F_shared:
        w["shared"] = synth.gen_shared(cfg)
        kw["shared"] = w["shared"]
        if cfg.shared_gate:
            w["w_sg"] = synth.gen_shared_gate(cfg)
            kw["w_shared_gate"] = w["w_sg"]
    if cfg.select_bias:
        w["select_bias"] = synth.gen_select_bias(cfg)
        kw["select_bias"] = w["select_bias"]
    step = MoELayer(cfg, router=w["router"], experts=w["experts"], device=DEV, **kw)
    calls = MoELayer(cfg, router=w["router"], experts=w["experts"], device=DEV, fused_step=False, **kw)
    return step, calls, w


def _same(a, b):
    if a is None or b is None:
        return a is None and b is None
    return torch.equal(a.contiguous().view(torch.uint8), b.contiguous().view(torch.uint8))


def _compare(step, calls, x, what):
    g = step.forward(x)
    ref = calls.forward(x)
    torch.cuda.synchronize()
    assert _same(g["out"], ref["out"]), f"{what}: output differs from the separate calls"
    for key in ROUTE_KEYS:
        assert _same(g["route"][key], ref["route"][key]), f"{what}: {key} differs from moe_route_permute"
    assert _same(g["route"]["shared_gate"], ref["route"]["shared_gate"]), f"{what}: shared gate differs"
    return g


@pytest.fixture(scope="module")
def qwen():
    cfg = synth.get_config("qwen_decode_bf16")
    step, calls, w = _layers(cfg, True)
    return cfg, step, calls, w


# 1-4 tokens fold the combine and split the shared down projection over K; 5 and 8 run the
# combine as its own launch; 16/17 cross into a second routing m-tile and into 16-row chunks of
# the shared expert; 64 is the largest step
@pytest.mark.parametrize("T", [1, 2, 4, 5, 8, 16, 17, 33, 64])
def test_qwen_step_bit_equal_to_separate_calls(qwen, T):
    cfg, step, calls, _ = qwen
    assert step.fused_decode_step(T) and not calls.fused_decode_step(T)
    for xi in (0, 1):
        _, x = _x(cfg, 40 + xi, T)
        say(f"  case qwen decode step T={T} x={xi}: launching")
        _compare(step, calls, x, f"qwen T={T} x={xi}")


@pytest.mark.parametrize("T", [1, 8, 64])
def test_qwen_step_against_oracle(qwen, T):
    cfg, step, _, w = qwen
    xs, x = _x(cfg, 50, T)
    say(f"  case qwen decode step vs oracle T={T}: launching")
    g = step.forward(x)
    torch.cuda.synchronize()
    check_exact_indices(cfg, g["route"], g["perm"], T)
    r_ref = oracle_route(cfg, xs, w["router"], w["w_sg"])
    same = route_agreement(cfg, r_ref, g["route"], key_tol=1e-4)
    toks = np.arange(T)[same]
    assert len(toks) >= max(1, T - 2), "the device's selection differs from the oracle's on too many tokens"
    need = sorted(set(r_ref.idx[toks].ravel().tolist()))
    ex = {e: oracle_expert(cfg, w["experts"][e]) for e in need}
    ref = moe.moe_layer(decode(xs, "bf16"), r_ref, lambda e: ex[e], cfg.E, shared=oracle_expert(cfg, w["shared"]),
                        tokens=toks)
    assert_close(to_np(g["out"])[toks], ref, "bf16", f"decode step T={T}")


def test_step_without_shared_expert():
    """The expert-offload layer's shape (E=128, top-8, d=4096) with every expert resident and no
    shared expert: the first launch only routes."""
    cfg = synth.get_config("offload_decode_bf16")
    step, calls, w = _layers(cfg, False)
    for T in (1, 8, 32, 64):
        xs, x = _x(cfg, 60, T)
        say(f"  case offload-shape decode step T={T}: launching")
        g = _compare(step, calls, x, f"no shared T={T}")
        check_exact_indices(cfg, g["route"], g["perm"], T)
    # the oracle on one step's first tokens
    r_ref = oracle_route(cfg, xs, w["router"])
    same = route_agreement(cfg, r_ref, g["route"], key_tol=1e-4)
    toks = np.arange(64)[same][:6]
    need = sorted(set(r_ref.idx[toks].ravel().tolist()))
    ex = {e: oracle_expert(cfg, w["experts"][e]) for e in need}
    ref = moe.moe_layer(decode(xs, "bf16"), r_ref, lambda e: ex[e], cfg.E, tokens=toks)
    assert_close(to_np(g["out"])[toks], ref, "bf16", "no shared, T=64")


def test_step_group_limited_sigmoid_routing():
    """DeepSeek-V3-style routing (sigmoid keys plus a per-expert selection bias, 8 groups, top-4
    groups by the sum of their top-2 keys, gates renormalised and scaled by 2.5) with a shared
    expert without a gate, at a reduced width in bf16."""
    cfg = synth.get_config("dsv3_prefill_fp8", dtype="bf16", d=512, F=256, F_shared=256)
    step, calls, w = _layers(cfg, True)
    for T in (1, 3, 16, 40):
        xs, x = _x(cfg, 70, T)
        say(f"  case grouped sigmoid decode step T={T}: launching")
        g = _compare(step, calls, x, f"grouped sigmoid T={T}")
        check_exact_indices(cfg, g["route"], g["perm"], T)
    r_ref = oracle_route(cfg, xs, w["router"], None, w["select_bias"])
    same = route_agreement(cfg, r_ref, g["route"], key_tol=1e-4)
    toks = np.arange(40)[same]
    need = sorted(set(r_ref.idx[toks].ravel().tolist()))
    ex = {e: oracle_expert(cfg, w["experts"][e]) for e in need}
    ref = moe.moe_layer(decode(xs, "bf16"), r_ref, lambda e: ex[e], cfg.E, shared=oracle_expert(cfg, w["shared"]),
                        tokens=toks)
    assert_close(to_np(g["out"])[toks], ref, "bf16", "grouped sigmoid, T=40")


def test_mxfp4_step_bit_equal_to_separate_calls():
    """MXFP4 bundles (codes and E8M0 scales decoded in registers) through the same three launches."""
    cfg = synth.get_config("qwen_decode_bf16", dtype="mxfp4")
    step, calls, _ = _layers(cfg, True)
    for T in (1, 4, 8, 64):
        _, x = _x(cfg, 80, T)
        say(f"  case mxfp4 decode step T={T}: launching")
        _compare(step, calls, x, f"mxfp4 T={T}")


def test_workspace_counters_return_to_zero_and_sizes_alternate(qwen):
    """One workspace through steps of changing size (64, 1, 17, 4, 64 tokens): each step equals the
    separate calls, and the routing's arrival counters are zero after every step."""
    cfg, step, calls, _ = qwen
    for i, T in enumerate((64, 1, 17, 4, 64)):
        _, x = _x(cfg, 90 + i, T)
        say(f"  case alternating sizes T={T}: launching")
        _compare(step, calls, x, f"alternating T={T}")
        ws = step._ws["step_ws"]
        assert int(ws[:256].count_nonzero()) == 0, "arrival counters left non-zero"


def test_step_graph_replays_match_eager(qwen):
    """The step captured as one HIP graph: every replay, with eager steps in between, equals the
    eager step on the same input bit for bit."""
    cfg, step, _, _ = qwen
    for T in (1, 8):
        _, x0 = _x(cfg, 100, T)
        x_static = x0.clone()
        graph, outs = step.capture(x_static)
        for i in range(4):
            _, xi = _x(cfg, 101 + i, T)
            x_static.copy_(xi)
            say(f"  case decode step graph T={T} replay {i}: launching")
            graph.replay()
            torch.cuda.synchronize()
            got = outs["out"].clone()
            eager = step.forward(xi)["out"]
            torch.cuda.synchronize()
            assert _same(got, eager), f"T={T} replay {i} differs from eager"
