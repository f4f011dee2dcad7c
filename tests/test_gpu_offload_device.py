"""The slot pool planned on the device (expert_slot_cache_dev): per step the device's hit and
miss tables equal the oracle's LRU simulation, outputs are bit-identical to every expert
resident and within tolerance of the oracle, a whole offload step replays as one captured
graph (routing, plan, copy kernel, expert FFN, combine) with every replay bit-identical to the
eager resident layer, and steps touching more experts than slots run in waves that refill the
same slots."""
import numpy as np
import pytest
import torch

from expert_offloaded_ffn_amd import synth
from expert_offloaded_ffn_amd.layer import MoELayer
from oracle import moe
from oracle.slot_cache import LRUSlotCache
from parity_util import assert_close, check_exact_indices, decode, oracle_expert, oracle_route, say, to_np

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _inputs(cfg, step):
    xs = synth.gen_x(cfg, step)
    x = torch.from_numpy(xs.view(np.int16)).view(torch.bfloat16).to(DEV)
    lb = synth.zipf_logit_bias(cfg, step)
    return xs, x, lb, torch.from_numpy(lb).to(DEV)


def _check_plan(layer, sim, idx):
    plan = sim.step(idx.ravel())
    E = layer.E
    hit_t, miss_t = to_np(layer.slot_table), to_np(layer.miss_slot_tables)
    want_hit = np.full(E, -1)
    want_miss = np.full(miss_t.shape, -1)
    assert len(plan.waves) <= miss_t.shape[0]
    for w, wave in enumerate(plan.waves):
        for en in wave:
            if en.hit:
                assert w == 0
                want_hit[en.expert] = en.slot
            else:
                want_miss[w, en.expert] = en.slot
    assert np.array_equal(hit_t, want_hit) and np.array_equal(miss_t, want_miss)


def _eager(cfg, steps, n_slots, oracle_every=0, freq_decay=0.0):
    router, experts = synth.gen_router(cfg), synth.gen_experts(cfg)
    layer = MoELayer(cfg, router=router, experts=experts, device=DEV, pool_slots=n_slots, device_plan=True,
                     freq_decay=freq_decay)
    resident = MoELayer(cfg, router=router, experts=experts, device=DEV)
    sim = LRUSlotCache(cfg.E, n_slots, freq_decay=freq_decay)
    oexp = {}
    for step in range(steps):
        xs, x, lb, lb_dev = _inputs(cfg, step)
        say(f"  case {cfg.name} E={cfg.E} slots={n_slots} device plan, step {step}: launching")
        g = layer.forward(x, logit_bias=lb_dev)
        ref = resident.forward(x, logit_bias=lb_dev)
        torch.cuda.synchronize()
        idx = check_exact_indices(cfg, g["route"], g["perm"], cfg.T)
        _check_plan(layer, sim, idx)
        out = to_np(g["out"])
        assert np.array_equal(out, to_np(ref["out"])), "device-planned pool differs from all-resident"
        if oracle_every and step % oracle_every == 0:
            r_ref = oracle_route(cfg, xs, router, logit_bias=lb)
            for e in set(r_ref.idx.ravel().tolist()) - oexp.keys():
                oexp[e] = oracle_expert(cfg, experts[e])
            assert_close(out, moe.moe_layer(decode(xs, "bf16"), r_ref, lambda e: oexp[e], cfg.E), "bf16")
    st = layer.cache_dev.stats()
    s = sim.stats
    assert (st["hits"], st["misses"], st["evictions"], st["steps"], st["waves"]) == \
        (s.hits, s.misses, s.evictions, s.steps, s.waves)
    assert st["h2d_bytes"] == s.misses * layer.bundle_bytes
    layer.cache_dev.close()
    return sim


def test_device_plan_small_parity():
    cfg = synth.get_config("offload_decode_bf16", E=16, d=256, F=256, T=3, k=4, zipf_epoch=4)
    sim = _eager(cfg, 12, 12, oracle_every=3)
    assert sim.stats.evictions > 0 and sim.stats.hits > 0


def test_device_plan_offload_shape():
    """The expert-offload shape with its own 32-slot pool: most steps need two or more waves."""
    cfg = synth.get_config("offload_decode_bf16")
    sim = _eager(cfg, 4, cfg.n_slots)
    assert sim.stats.misses > 0 and sim.stats.waves > sim.stats.steps


def test_device_plan_frequency_victims():
    """Frequency-aware victims on the device: the same plans as the oracle, single and multi-wave."""
    small = synth.get_config("offload_decode_bf16", E=16, d=256, F=256, T=8, k=4, zipf_epoch=6)
    sim = _eager(small, 12, 5, oracle_every=4, freq_decay=0.8)
    assert sim.stats.evictions > 0 and sim.stats.waves > sim.stats.steps
    full = synth.get_config("offload_decode_bf16")
    sim = _eager(full, 6, full.n_slots, freq_decay=0.8)
    assert sim.stats.hits > 0


def test_device_plan_waves_reuse_slots():
    """8 experts, 2 slots: every step runs several waves through the same two slots."""
    cfg = synth.get_config("offload_decode_bf16", E=8, d=256, F=512, T=16, k=2, zipf_alpha=0.0, zipf_epoch=64)
    sim = _eager(cfg, 6, 2, oracle_every=2)
    assert sim.stats.waves >= 3 * 6


def test_device_plan_whole_step_graph():
    cfg = synth.get_config("offload_decode_bf16", E=16, d=256, F=512, T=3, k=4, zipf_epoch=3)
    router, experts = synth.gen_router(cfg), synth.gen_experts(cfg)
    layer = MoELayer(cfg, router=router, experts=experts, device=DEV, pool_slots=5, device_plan=True)
    resident = MoELayer(cfg, router=router, experts=experts, device=DEV)
    sim = LRUSlotCache(cfg.E, 5)
    xs0, x0, lb0, lb0_dev = _inputs(cfg, 0)
    x_static, lb_static = x0.clone(), lb0_dev.clone()
    say("  case device-plan graph: capture")
    graph, outs = layer.capture(x_static, lb_static)
    # the captured outputs hold nothing until a replay; the resident layer routes identically
    idx0 = to_np(resident.forward(x0, logit_bias=lb0_dev)["route"]["idx"])
    torch.cuda.synchronize()
    sim.step(idx0.ravel())            # capture() runs two real warm-up steps on step 0's inputs
    sim.step(idx0.ravel())
    for step in range(1, 10):
        xs, x, lb, lb_dev = _inputs(cfg, step)
        x_static.copy_(x)
        lb_static.copy_(lb_dev)
        say(f"  case device-plan graph: replay {step}")
        graph.replay()
        ref = resident.forward(x, logit_bias=lb_dev)
        torch.cuda.synchronize()
        idx = check_exact_indices(cfg, outs["route"], outs["perm"], cfg.T)
        _check_plan(layer, sim, idx)
        assert np.array_equal(to_np(outs["out"]), to_np(ref["out"])), f"replay {step} differs from eager resident"
    st = layer.cache_dev.stats()
    assert (st["hits"], st["misses"], st["evictions"], st["steps"], st["waves"]) == \
        (sim.stats.hits, sim.stats.misses, sim.stats.evictions, sim.stats.steps, sim.stats.waves)
    assert sim.stats.misses > cfg.E // 2 and sim.stats.waves > sim.stats.steps   # loads, and multi-wave steps
    layer.cache_dev.close()


