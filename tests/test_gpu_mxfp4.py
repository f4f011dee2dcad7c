"""MXFP4 expert weights (FP4 E2M1 codes with an E8M0 scale per 32 inputs) through the decode
kernels, against the float64 oracle on the decoded weights: resident layers at reduced and at
full offload-workload size, and the expert slot pool."""
import numpy as np
import pytest
import torch

from expert_offloaded_ffn_amd import binding as B
from expert_offloaded_ffn_amd import synth
from expert_offloaded_ffn_amd.layer import MoELayer
from oracle import moe
from parity_util import (assert_close, check_exact_indices, decode, oracle_expert, oracle_route, route_agreement,
                         say, to_np)

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _x(cfg, xs):
    return torch.from_numpy(xs.view(np.int16)).view(torch.bfloat16).to(DEV)


def _check(cfg, layer, router, experts, T, xi, logit_bias=None, tokens=None):
    xs = synth.gen_x(cfg, xi, T=T)
    lb = None if logit_bias is None else torch.from_numpy(logit_bias).to(DEV)
    say(f"  case {cfg.name} T={T} x={xi}: launching")
    g = layer.forward(_x(cfg, xs), logit_bias=lb)
    torch.cuda.synchronize()
    say("    done")
    check_exact_indices(cfg, g["route"], g["perm"], T)
    r_ref = oracle_route(cfg, xs, router, logit_bias=logit_bias)
    same = route_agreement(cfg, r_ref, g["route"], key_tol=1e-4)
    toks = np.arange(T) if tokens is None else np.asarray(tokens)
    toks = toks[same[toks]]
    cache = {}

    def expert(e):
        if e not in cache:
            cache[e] = oracle_expert(cfg, experts[e])
        return cache[e]

    ref = moe.moe_layer(decode(xs, "bf16"), r_ref, expert, cfg.E, tokens=toks)
    assert_close(to_np(g["out"])[toks], ref, "bf16", f"{cfg.name} T={T}")
    return g


@pytest.mark.parametrize("T,d,E,k,F", [(1, 256, 16, 4, 256), (5, 256, 16, 4, 384), (32, 512, 32, 8, 256),
                                       (64, 256, 8, 2, 128)])
def test_mxfp4_decode_layer_reduced(T, d, E, k, F):
    cfg = synth.get_config("offload_decode_mxfp4", T=T, d=d, E=E, k=k, F=F, name=f"mxfp4_T{T}_d{d}_E{E}_k{k}_F{F}")
    router, experts = synth.gen_router(cfg), synth.gen_experts(cfg)
    layer = MoELayer(cfg, router=router, experts=experts, device=DEV)
    for xi in range(2):
        _check(cfg, layer, router, experts, T, xi)


def test_mxfp4_offload_workload_resident():
    """The full offload workload shape (E=128, d=4096, F=1536, top-8, T=32) with every expert
    resident, under the Zipf prior of step 0."""
    cfg = synth.get_config("offload_decode_mxfp4")
    router, experts = synth.gen_router(cfg), synth.gen_experts(cfg, threads=16)
    layer = MoELayer(cfg, router=router, experts=experts, device=DEV, threads=16)
    _check(cfg, layer, router, experts, cfg.T, 0, logit_bias=synth.zipf_logit_bias(cfg, 0), tokens=[0, 7, 31])


def test_mxfp4_slot_pool_matches_resident():
    """MXFP4 bundles through the expert slot pool (8 slots for 32 experts): every step equals the
    resident layer bit for bit, and the hit/miss counts follow the pool."""
    cfg = synth.get_config("offload_decode_mxfp4", d=512, F=256, E=32, k=4, T=16, n_slots=8)
    router, experts = synth.gen_router(cfg), synth.gen_experts(cfg)
    res = MoELayer(cfg, router=router, experts=experts, device=DEV)
    pool = MoELayer(cfg, router=router, experts=experts, device=DEV, pool_slots=cfg.n_slots)
    for step in range(6):
        x = _x(cfg, synth.gen_x(cfg, step))
        lb = torch.from_numpy(synth.zipf_logit_bias(cfg, step)).to(DEV)
        say(f"  case mxfp4 slot pool step {step}: launching")
        a = res.forward(x, logit_bias=lb)["out"]
        b = pool.forward(x, logit_bias=lb)["out"]
        torch.cuda.synchronize()
        say("    done")
        assert torch.equal(a.view(torch.int16), b.view(torch.int16)), f"step {step}"
    st = pool.cache.stats()
    assert st["misses"] > 0 and st["h2d_bytes"] == st["misses"] * B.bundle_bytes(cfg.d, cfg.F, B.MOE_MXFP4)
    pool.cache.close()


@pytest.mark.parametrize("T", [1, 3, 8, 40])
def test_mxfp4_with_shared_expert(T):
    """A Qwen1.5-MoE-shaped layer (E=60 top-4, F=1408, gated shared expert F=5632) with MXFP4
    weights: the shared expert runs in the routed experts' decode launches (and, for 1-4 tokens,
    the combine in the down launch); against the oracle."""
    cfg = synth.get_config("qwen_decode_bf16", dtype="mxfp4", T=T, name=f"qwen_mxfp4_T{T}")
    router, experts, shared = synth.gen_router(cfg), synth.gen_experts(cfg), synth.gen_shared(cfg)
    w_sg = synth.gen_shared_gate(cfg)
    layer = MoELayer(cfg, router=router, experts=experts, shared=shared, w_shared_gate=w_sg, device=DEV)
    assert layer.shared_in_decode_launch(T)
    xs = synth.gen_x(cfg, 0, T=T)
    say(f"  case {cfg.name}: launching")
    g = layer.forward(_x(cfg, xs))
    torch.cuda.synchronize()
    say("    done")
    check_exact_indices(cfg, g["route"], g["perm"], T)
    r_ref = oracle_route(cfg, xs, router, w_sg)
    same = route_agreement(cfg, r_ref, g["route"], key_tol=1e-4)
    toks = np.arange(T)[same]
    ref = moe.moe_layer(decode(xs, "bf16"), r_ref, lambda e: oracle_expert(cfg, experts[e]), cfg.E,
                        shared=oracle_expert(cfg, shared), tokens=toks)
    assert_close(to_np(g["out"])[toks], ref, "bf16", cfg.name)


def test_mxfp4_fused_combine_bit_equal():
    """moe_grouped_ffn_combine on MXFP4 problems equals the batch call plus moe_combine."""
    cfg = synth.get_config("offload_decode_mxfp4", d=512, F=256, E=32, k=4, T=12)
    layer = MoELayer(cfg, router=synth.gen_router(cfg), experts=synth.gen_experts(cfg), device=DEV)
    x = _x(cfg, synth.gen_x(cfg, 0))
    p = B.route_permute(x, layer.w_router_t, **layer.route_args())
    rows = cfg.T * cfg.k
    pr = B.ffn_problem(layer.table, rows, p["offsets"], x, a_row_src=p["perm_src"], a_row_div=cfg.k)
    y = B.grouped_ffn_batch([pr])[0]
    ref = B.combine(y, p["perm_dst"], p["gate"])
    pr2 = B.ffn_problem(layer.table, rows, p["offsets"], x, a_row_src=p["perm_src"], a_row_div=cfg.k)
    say("  case mxfp4 fused combine: launching")
    got = B.grouped_ffn_combine(pr2, None, p["perm_dst"], p["gate"])
    torch.cuda.synchronize()
    say("    done")
    assert torch.equal(got.view(torch.int16), ref.view(torch.int16))


# ------------------------------------------------ prefill: block-scaled MFMA --
# More than 64 tokens: activations and hidden activations in MXFP8 (E4M3 with a power-of-two
# scale per 32, the OCP MX conversion), MXFP4 weights on v_mfma_scale_f32_16x16x128_f8f6f4.

def test_permute_mxfp8_quantisation_bit_exact():
    """moe_permute's MXFP8 output (token order and gathered) equals the oracle's OCP MX
    conversion code for code and exponent for exponent."""
    from oracle import formats
    cfg = synth.get_config("offload_decode_mxfp4", T=200, d=512, E=16, k=4)
    rng = np.random.default_rng(3)
    idx = np.stack([rng.choice(cfg.E, cfg.k, replace=False) for _ in range(cfg.T)]).astype(np.int32)
    xs = synth.gen_x(cfg, 0)
    xs[7, 32:64] = 0          # an all-zero block
    x = _x(cfg, xs)
    say("  case permute mxfp8: launching")
    tok = B.permute(torch.from_numpy(idx).to(DEV), cfg.E, x=x, out_dtype=B.MOE_MXFP8, gather=0)
    gat = B.permute(torch.from_numpy(idx).to(DEV), cfg.E, x=x, out_dtype=B.MOE_MXFP8, gather=1)
    torch.cuda.synchronize()
    codes, exps = formats.quantize_rows_mxfp8(decode(xs, "bf16"))
    assert np.array_equal(to_np(tok["x_out"]), codes)
    assert np.array_equal(to_np(tok["x_out_scale"]), exps)
    src = to_np(gat["perm_src"]) // cfg.k
    assert np.array_equal(to_np(gat["x_out"]), codes[src])
    assert np.array_equal(to_np(gat["x_out_scale"]), exps[src])
    assert exps[7, 1] == 0


def _check_prefill(cfg, layer, router, experts, T, xi, shared=None, w_sg=None, tokens=None):
    xs = synth.gen_x(cfg, xi, T=T)
    say(f"  case {cfg.name} T={T} x={xi} (MXFP4 prefill): launching")
    g = layer.forward(_x(cfg, xs))
    torch.cuda.synchronize()
    say("    done")
    check_exact_indices(cfg, g["route"], g["perm"], T)
    r_ref = oracle_route(cfg, xs, router, w_sg)
    same = route_agreement(cfg, r_ref, g["route"], key_tol=1e-4)
    toks = np.arange(T) if tokens is None else np.asarray(tokens)
    toks = toks[same[toks]]
    cache = {}

    def expert(e):
        if e not in cache:
            cache.clear()
            cache[e] = oracle_expert(cfg, experts[e])
        return cache[e]

    ref = moe.moe_layer(decode(xs, "bf16"), r_ref, expert, cfg.E, quant_act="mxfp8", tokens=toks,
                        shared=None if shared is None else oracle_expert(cfg, shared))
    assert_close(to_np(g["out"])[toks], ref, "bf16", f"{cfg.name} T={T}")
    return g


@pytest.mark.parametrize("T,d,E,k,F", [(65, 256, 8, 2, 128), (300, 512, 8, 2, 512), (600, 256, 16, 4, 768),
                                       (100, 512, 32, 8, 256)])
def test_mxfp4_prefill_layer_reduced(T, d, E, k, F):
    cfg = synth.get_config("offload_decode_mxfp4", T=T, d=d, E=E, k=k, F=F, name=f"mxfp4p_T{T}_d{d}_E{E}_k{k}_F{F}")
    router, experts = synth.gen_router(cfg), synth.gen_experts(cfg)
    layer = MoELayer(cfg, router=router, experts=experts, device=DEV)
    assert layer.mx_prefill(T)
    _check_prefill(cfg, layer, router, experts, T, 0)


def test_mxfp4_prefill_many_tiles_every_row():
    """512 gate/up tiles (16 experts x 2 m-tiles x 16 n-tiles), more than the persistent grid,
    so blocks run several tiles through the 3-stage ring; every row checked."""
    cfg = synth.get_config("offload_decode_mxfp4", T=2048, d=512, E=16, k=4, F=2048, name="mxfp4p_many_tiles")
    router, experts = synth.gen_router(cfg), synth.gen_experts(cfg)
    layer = MoELayer(cfg, router=router, experts=experts, device=DEV)
    g = _check_prefill(cfg, layer, router, experts, cfg.T, 1)
    assert to_np(g["route"]["counts"]).max() > 256


def test_mxfp4_prefill_offload_shape():
    """The offload workload's experts (d=4096, E=128 top-8, F=1536) at 512 tokens, resident."""
    cfg = synth.get_config("offload_decode_mxfp4", T=512)
    router, experts = synth.gen_router(cfg), synth.gen_experts(cfg, threads=16)
    layer = MoELayer(cfg, router=router, experts=experts, device=DEV)
    rng = np.random.default_rng(4)
    _check_prefill(cfg, layer, router, experts, cfg.T, 2, tokens=np.sort(rng.choice(cfg.T, 96, replace=False)))


def test_mxfp4_prefill_with_folded_shared_expert():
    """A Qwen1.5-MoE-shaped layer with MXFP4 weights at 160 tokens: the shared expert is one more
    group of the routed experts' block-scaled launches; against the oracle (sigmoid shared gate)."""
    cfg = synth.get_config("qwen_decode_bf16", dtype="mxfp4", T=160, name="qwen_mxfp4_prefill")
    router, experts, shared = synth.gen_router(cfg), synth.gen_experts(cfg), synth.gen_shared(cfg)
    w_sg = synth.gen_shared_gate(cfg)
    layer = MoELayer(cfg, router=router, experts=experts, shared=shared, w_shared_gate=w_sg, device=DEV)
    assert layer.shared_in_routed_launch(cfg.T)
    _check_prefill(cfg, layer, router, experts, cfg.T, 3, shared=shared, w_sg=w_sg)


def test_mxfp4_prefill_slot_pool_matches_resident():
    """The slot pool (8 of 32 experts) running MXFP4 prefill steps in waves gives the resident
    layer's output bit for bit."""
    cfg = synth.get_config("offload_decode_mxfp4", d=512, F=256, E=32, k=4, T=96, n_slots=8)
    router, experts = synth.gen_router(cfg), synth.gen_experts(cfg)
    res = MoELayer(cfg, router=router, experts=experts, device=DEV)
    pool = MoELayer(cfg, router=router, experts=experts, device=DEV, pool_slots=8)
    for step in range(3):
        x = _x(cfg, synth.gen_x(cfg, step))
        say(f"  case mxfp4 prefill slot pool step {step}: launching")
        a = res.forward(x)["out"]
        g = pool.forward(x)
        torch.cuda.synchronize()
        assert g["waves"] >= 2
        assert torch.equal(a.view(torch.int16), g["out"].view(torch.int16))
    pool.cache.close()
