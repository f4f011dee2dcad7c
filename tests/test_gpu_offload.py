"""The expert slot pool on the GPU: per-step plans and statistics equal the oracle's
LRU simulation exactly (given the device's routing), outputs equal the oracle's layer,
blocking and overlapped modes give bit-identical outputs, and slots reused across
waves within a step never expose a half-copied bundle."""
import numpy as np
import pytest
import torch

from expert_offloaded_ffn_amd import synth
from expert_offloaded_ffn_amd.layer import MoELayer
from oracle import moe
from oracle.slot_cache import LRUSlotCache
from parity_util import (assert_close, check_exact_indices, decode, oracle_expert, oracle_route, route_agreement, say,
                         to_np)

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _x(cfg, step):
    xs = synth.gen_x(cfg, step)
    return xs, torch.from_numpy(xs.view(np.int16)).view(torch.bfloat16).to(DEV)


def _run(cfg, steps, *, n_slots, blocking=False, check_outputs=True, tokens=None, freq_decay=0.0):
    router = synth.gen_router(cfg)
    experts = synth.gen_experts(cfg)
    layer = MoELayer(cfg, router=router, experts=experts, device=DEV, pool_slots=n_slots, blocking=blocking,
                     freq_decay=freq_decay)
    sim = LRUSlotCache(cfg.E, n_slots, freq_decay=freq_decay)
    outs = []
    ocache = {}

    def expert(e):
        if e not in ocache:
            ocache[e] = oracle_expert(cfg, experts[e])
        return ocache[e]

    for step in range(steps):
        xs, x = _x(cfg, step)
        lb = synth.zipf_logit_bias(cfg, step)
        say(f"  case {cfg.name} slots={n_slots} blocking={blocking} step={step}: launching")
        g = layer.forward(x, logit_bias=torch.from_numpy(lb).to(DEV))
        torch.cuda.synchronize()
        idx = check_exact_indices(cfg, g["route"], g["perm"], cfg.T)
        plan = sim.step(idx.ravel())
        assert g["waves"] == len(plan.waves)
        for w, wave in enumerate(plan.waves):
            assert layer.cache.wave_plan(w) == [(en.expert, en.slot, int(en.hit), en.evicted) for en in wave]
        st = layer.cache.stats()
        assert (st["hits"], st["misses"], st["evictions"], st["waves"]) == \
            (sim.stats.hits, sim.stats.misses, sim.stats.evictions, sim.stats.waves)
        assert st["h2d_bytes"] == sim.stats.misses * layer.bundle_bytes
        out = to_np(g["out"])
        outs.append(out.copy())
        if check_outputs:
            r_ref = oracle_route(cfg, xs, router, logit_bias=lb)
            same = route_agreement(cfg, r_ref, g["route"], key_tol=1e-4)
            toks = np.arange(cfg.T) if tokens is None else np.asarray(tokens)
            toks = toks[same[toks]]
            ref = moe.moe_layer(decode(xs, "bf16"), r_ref, expert, cfg.E, tokens=toks)
            assert_close(out[toks], ref, "bf16")
    layer.cache.close()
    return outs, sim


def test_slot_pool_small_parity_and_plans():
    cfg = synth.get_config("offload_decode_bf16", E=16, d=256, F=256, T=8, k=4, zipf_epoch=4, n_slots=4)
    outs, sim = _run(cfg, 12, n_slots=4)
    assert sim.stats.evictions > 0 and sim.stats.hits > 0


def test_blocking_and_overlapped_modes_agree_bitwise():
    cfg = synth.get_config("offload_decode_bf16", E=16, d=256, F=256, T=8, k=4, zipf_epoch=4, n_slots=4)
    a, _ = _run(cfg, 8, n_slots=4, blocking=False, check_outputs=False)
    b, _ = _run(cfg, 8, n_slots=4, blocking=True, check_outputs=False)
    for x, y in zip(a, b):
        assert np.array_equal(x, y)


def test_two_slots_reused_across_waves_every_step():
    """8 experts, 2 slots: every step runs several waves that refill the same two slots, so a
    copy must wait for the previous wave's kernels before overwriting a slot."""
    cfg = synth.get_config("offload_decode_bf16", E=8, d=256, F=512, T=16, k=2, zipf_alpha=0.0, zipf_epoch=64)
    outs, sim = _run(cfg, 6, n_slots=2)
    assert sim.stats.waves >= 3 * 6


def test_offload_full_size_few_steps():
    cfg = synth.get_config("offload_decode_bf16")
    outs, sim = _run(cfg, 4, n_slots=cfg.n_slots, tokens=[0, 7, 13, 31])
    assert sim.stats.misses > 0


def test_frequency_victims_plans_and_parity():
    """Frequency-aware victims: every step's plan equals the oracle's, outputs match the oracle."""
    cfg = synth.get_config("offload_decode_bf16", E=16, d=256, F=256, T=8, k=4, zipf_epoch=6, n_slots=5)
    outs, sim = _run(cfg, 12, n_slots=5, freq_decay=0.8)
    assert sim.stats.evictions > 0 and sim.stats.hits > 0
