"""The decode FFN with the combine folded into its down launch (moe_grouped_ffn_combine),
through the C ABI: bit-equal to the grouped FFN batch followed by moe_combine, and within the
bf16 tolerance of the float64 oracle."""
import numpy as np
import pytest
import torch

from expert_offloaded_ffn_amd import binding as B
from expert_offloaded_ffn_amd import synth
from expert_offloaded_ffn_amd import layer as layer_mod
from expert_offloaded_ffn_amd.layer import MoELayer
from oracle import moe
from parity_util import assert_close, decode, oracle_expert, oracle_route, route_agreement, say, to_np

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _x(cfg, xi, T):
    return torch.from_numpy(synth.gen_x(cfg, xi, T=T).view(np.int16)).view(torch.bfloat16).to(DEV)


@pytest.fixture(scope="module")
def qwen():
    cfg = synth.get_config("qwen_decode_bf16")
    w = dict(router=synth.gen_router(cfg), experts=synth.gen_experts(cfg), shared=synth.gen_shared(cfg),
             w_sg=synth.gen_shared_gate(cfg))
    # the separate calls (fused_step=False): this module tests moe_grouped_ffn_combine
    layer = MoELayer(cfg, router=w["router"], experts=w["experts"], shared=w["shared"], w_shared_gate=w["w_sg"],
                     device=DEV, fused_step=False)
    return cfg, layer, w


# 1-4 tokens split the shared expert's down projection over K; 16 / 17 switch the m-block
# variant; 64 is the largest decode batch
@pytest.mark.parametrize("T", [1, 3, 4, 8, 16, 17, 40, 64])
def test_fused_combine_bit_equal_to_two_calls(qwen, T):
    cfg, layer, _ = qwen
    old_max = layer_mod.FUSE_COMBINE_MAX_T
    layer_mod.FUSE_COMBINE_MAX_T = 64   # every decode batch size through the fused call
    try:
        for xi in (0, 1):
            x = _x(cfg, 20 + xi, T)
            say(f"  case qwen fused combine T={T} x={xi}: launching")
            layer.fuse_combine = False
            ref = layer.forward(x)["out"].clone()
            layer.fuse_combine = True
            got = layer.forward(x)["out"].clone()
            torch.cuda.synchronize()
            say("    done")
            assert torch.equal(got.view(torch.int16), ref.view(torch.int16)), f"T={T} x={xi}: fused != two calls"
    finally:
        layer_mod.FUSE_COMBINE_MAX_T = old_max


@pytest.mark.parametrize("T", [1, 3, 4])
def test_fused_combine_against_oracle(qwen, T):
    cfg, layer, w = qwen
    layer.fuse_combine = True
    if T > layer_mod.FUSE_COMBINE_MAX_T:
        pytest.skip("the layer combines in its own launch at this batch size")
    x_store = synth.gen_x(cfg, 30, T=T)
    x = torch.from_numpy(x_store.view(np.int16)).view(torch.bfloat16).to(DEV)
    say(f"  case qwen fused combine vs oracle T={T}: launching")
    g = layer.forward(x)
    torch.cuda.synchronize()
    say("    done")
    r_ref = oracle_route(cfg, x_store, w["router"], w["w_sg"], None, None)
    same = route_agreement(cfg, r_ref, g["route"], key_tol=1e-4)
    toks = np.arange(T)[same]
    cache = {}

    def expert(e):
        if e not in cache:
            cache.clear()
            cache[e] = oracle_expert(cfg, w["experts"][e])
        return cache[e]

    ref = moe.moe_layer(decode(x_store, "bf16"), r_ref, expert, cfg.E, shared=oracle_expert(cfg, w["shared"]),
                        tokens=toks)
    assert_close(to_np(g["out"])[toks], ref, "bf16", f"fused T={T}")


def _routed_problem(layer, p, x, k, y_dtype):
    return B.ffn_problem(layer.table, x.shape[0] * k, p["offsets"], x, a_row_src=p["perm_src"], a_row_div=k,
                         y_dtype=y_dtype)


@pytest.mark.parametrize("name,over,T,ydt,odt", [
    ("mixtral_prefill_bf16", dict(d=256, F=512, E=40, k=12), 9, B.MOE_BF16, B.MOE_BF16),   # k > 8, no shared
    ("mixtral_prefill_bf16", dict(d=256, F=512), 5, B.MOE_F32, B.MOE_F32),                 # fp32 y and out
    ("offload_decode_bf16", dict(d=512, F=256), 32, B.MOE_BF16, B.MOE_F32),                # E = 128, top-8
])
def test_fused_combine_without_shared_expert(name, over, T, ydt, odt):
    """Only a routed problem: bit-equal to moe_grouped_ffn + moe_combine with the same y and out dtypes."""
    cfg = synth.get_config(name, **over)
    layer = MoELayer(cfg, router=synth.gen_router(cfg), experts=synth.gen_experts(cfg), device=DEV)
    for xi in (0, 1, 2):
        x = _x(cfg, xi, T)
        say(f"  case {cfg.name} routed-only fused T={T} x={xi}: launching")
        p = B.route_permute(x, layer.w_router_t, **layer.route_args())
        pr = _routed_problem(layer, p, x, cfg.k, ydt)
        y = B.grouped_ffn_batch([pr])[0]
        ref = B.combine(y, p["perm_dst"], p["gate"], out_dtype=odt)
        pr2 = _routed_problem(layer, p, x, cfg.k, ydt)
        got = B.grouped_ffn_combine(pr2, None, p["perm_dst"], p["gate"], out_dtype=odt)
        torch.cuda.synchronize()
        say("    done")
        view = torch.int16 if odt == B.MOE_BF16 else torch.int32
        assert torch.equal(got.view(view), ref.view(view)), f"{cfg.name} x={xi}: fused != two calls"


def test_fused_combine_graph_replays(qwen):
    """Captured in a HIP graph, the fused decode step's replays equal eager forward calls (the
    group counts are cleared by the gate/up launch inside the graph, not by a memset)."""
    cfg, layer, _ = qwen
    layer.fuse_combine = True
    T = 2
    x_static = _x(cfg, 40, T)
    say("  case qwen fused combine graph: capture")
    graph, outs = layer.capture(x_static)
    for i in range(4):
        xi = _x(cfg, 41 + i, T)
        x_static.copy_(xi)
        graph.replay()
        torch.cuda.synchronize()
        got = outs["out"].clone()
        ref = layer.forward(xi)["out"]
        torch.cuda.synchronize()
        assert torch.equal(got.view(torch.int16), ref.view(torch.int16)), f"replay {i} differs from eager"
    say("    done")
