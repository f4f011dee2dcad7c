"""The slot pool's executor under stress: a slot reused by a later wave while the previous
wave's kernels are held back, a bundle copy that fails, a reset followed by a re-run, the
compute stream's wait statistic, and a device-planned pool under a layer with a shared expert.

The pages' cache blocks on a wave's transfers and refuses to run on an incomplete bundle
("Running 35B MoE Models on 8GB GPUs: How vvllm-ms Caches Experts in System RAM", section
"Technical Insight"); these tests force the situations in which that could go wrong. The
delays are bounded spin kernels (torch.cuda._sleep) and the copy failure is injected on the
host (MOEFFN_FAIL_COPY_AT), so every kernel still ends normally."""
import os

import numpy as np
import pytest
import torch

from expert_offloaded_ffn_amd import binding as B
from expert_offloaded_ffn_amd import synth
from expert_offloaded_ffn_amd.layer import MoELayer
from oracle import moe
from oracle.slot_cache import LRUSlotCache
from parity_util import assert_close, check_exact_indices, decode, oracle_expert, oracle_route, say, to_np

pytestmark = pytest.mark.gpu
DEV = "cuda"
SPIN_CYCLES = 20_000_000   # about 10 ms at the shader clock: far longer than a small wave's copies


def _x(cfg, step):
    xs = synth.gen_x(cfg, step)
    return xs, torch.from_numpy(xs.view(np.int16)).view(torch.bfloat16).to(DEV)


def _pool_step(layer, x, lb, delay=0):
    """One forward of a host-planned slot-pool layer written out call by call, with a bounded
    spin kernel on the compute stream before every grouped-FFN launch of every wave part when
    `delay` is set: the kernels that read a slot then start long after the host has issued the
    next wave's copies into the same slots, so only the copies' wait for the slot's last read
    keeps the output right."""
    main = torch.cuda.current_stream()
    r = p = B.route_permute(x, layer.w_router_t, logit_bias=lb, ws=layer._buf("perm_ws", B.route_permute_workspace_size(
        x.shape[0], layer.k, layer.E, layer.d)), stream=main, **layer.route_args())
    rows = x.shape[0] * layer.k
    y = torch.empty(rows, layer.d, device=DEV, dtype=torch.bfloat16)
    fws = layer._buf("ffn_ws", B.grouped_ffn_workspace_size(layer.table, rows, B.MOE_BF16))
    waves = layer.cache.acquire(r["counts"], stream=main)
    for w in range(waves):
        for part in (0, 1):
            if layer.cache.wave(w, part, layer.slot_table, stream=main):
                if delay:
                    torch.cuda._sleep(delay)
                B.grouped_ffn(layer.table, rows, p["offsets"], x, act_dtype=B.MOE_BF16, a_row_src=p["perm_src"],
                              a_row_div=layer.k, y=y, y_dtype=B.MOE_BF16, ws=fws, stream=main)
        layer.cache.release(w, stream=main)
    out = B.combine(y, p["perm_dst"], r["gate"], stream=main)
    return out, waves


def test_slot_reuse_waits_for_delayed_kernels():
    """8 experts, 2 slots, 16 tokens at top-2: every step runs four waves through the same two
    slots. The kernels of each wave are held back by a spin kernel, so a copy that did not wait
    for the previous wave's last read would overwrite a bundle before it is read."""
    cfg = synth.get_config("offload_decode_bf16", E=8, d=256, F=512, T=16, k=2, zipf_alpha=0.0, zipf_epoch=64)
    router, experts = synth.gen_router(cfg), synth.gen_experts(cfg)
    for blocking in (False, True):
        layer = MoELayer(cfg, router=router, experts=experts, device=DEV, pool_slots=2, blocking=blocking)
        resident = MoELayer(cfg, router=router, experts=experts, device=DEV)
        total_waves = 0
        for step in range(4):
            xs, x = _x(cfg, step)
            say(f"  case delayed slot reuse blocking={blocking} step={step}: launching")
            out, waves = _pool_step(layer, x, None, delay=SPIN_CYCLES)
            ref = resident.forward(x)["out"]
            torch.cuda.synchronize()
            total_waves += waves
            assert torch.equal(out.view(torch.int16), ref.view(torch.int16)), f"step {step}: output differs"
        assert total_waves >= 3 * 4
        st = layer.cache.stats()
        assert st["misses"] > 0 and st["wait_ms"] >= 0.0
        layer.cache.close()


def test_copy_failure_is_loud_and_leaves_the_pool_consistent():
    """The 3rd bundle copy fails (injected on the host). The step raises MOE_EHIP, the expert
    whose copy failed and every miss not yet copied leave the residency table, and the next
    steps plan them as misses again and compute the same outputs as every expert resident.
    One token at top-4 over 4 slots: the failing step is a single wave of 4 misses."""
    cfg = synth.get_config("offload_decode_bf16", E=16, d=256, F=256, T=1, k=4, zipf_epoch=4, n_slots=4)
    router, experts = synth.gen_router(cfg), synth.gen_experts(cfg)
    os.environ["MOEFFN_FAIL_COPY_AT"] = "3"
    try:
        layer = MoELayer(cfg, router=router, experts=experts, device=DEV, pool_slots=4)
    finally:
        del os.environ["MOEFFN_FAIL_COPY_AT"]
    resident = MoELayer(cfg, router=router, experts=experts, device=DEV)
    xs, x = _x(cfg, 0)
    lb = torch.from_numpy(synth.zipf_logit_bias(cfg, 0)).to(DEV)
    say("  case injected copy failure: launching the failing step")
    with pytest.raises(RuntimeError) as ei:
        layer.forward(x, logit_bias=lb)
    assert "failed" in str(ei.value)
    torch.cuda.synchronize()
    # the failing step's one wave had 4 misses: copies 1 and 2 were issued, copy 3 failed, so
    # exactly two experts stay resident and the next identical step hits on them
    st0 = layer.cache.stats()
    assert st0["h2d_bytes"] == 2 * layer.bundle_bytes
    with pytest.raises(RuntimeError):
        layer.cache.wave(0, 0, layer.slot_table)      # the failed step has ended
    for step in range(5):
        xs, x = _x(cfg, step)
        lb = torch.from_numpy(synth.zipf_logit_bias(cfg, step)).to(DEV)
        say(f"  case after the failure, step {step}: launching")
        g = layer.forward(x, logit_bias=lb)
        ref = resident.forward(x, logit_bias=lb)
        torch.cuda.synchronize()
        assert torch.equal(g["out"].view(torch.int16), ref["out"].view(torch.int16)), f"step {step} differs"
        if step == 0:
            assert g["waves"] == 1
            plan = layer.cache.wave_plan(0)
            assert len(plan) == 4 and sum(en[2] for en in plan) == 2, "exactly the two copied experts are hits"
    layer.cache.close()


def test_reset_then_rerun_is_bit_identical():
    """Six steps, reset, the same six steps: identical plans, statistics and output bits."""
    cfg = synth.get_config("offload_decode_bf16", E=16, d=256, F=256, T=8, k=4, zipf_epoch=3, n_slots=5)
    router, experts = synth.gen_router(cfg), synth.gen_experts(cfg)
    layer = MoELayer(cfg, router=router, experts=experts, device=DEV, pool_slots=5)
    runs = []
    for run in range(2):
        outs, plans = [], []
        for step in range(6):
            xs, x = _x(cfg, step)
            lb = torch.from_numpy(synth.zipf_logit_bias(cfg, step)).to(DEV)
            say(f"  case reset re-run {run} step {step}: launching")
            g = layer.forward(x, logit_bias=lb)
            torch.cuda.synchronize()
            outs.append(g["out"].view(torch.int16).cpu().clone())
            plans.append([layer.cache.wave_plan(w) for w in range(g["waves"])])
        st = layer.cache.stats()
        runs.append((outs, plans, {k: st[k] for k in ("steps", "hits", "misses", "evictions", "waves", "h2d_bytes")}))
        layer.cache.reset()
    (o1, p1, s1), (o2, p2, s2) = runs
    assert s1 == s2 and p1 == p2
    assert all(torch.equal(a, b) for a, b in zip(o1, o2))
    assert s1["misses"] > 0 and s1["evictions"] > 0
    layer.cache.close()


def test_wait_stat_in_blocking_mode():
    """In blocking mode a wave's copies start only after all compute enqueued before them, so the
    compute stream waits for every wave that has misses: wait_ms is positive and at most the
    run's span."""
    cfg = synth.get_config("offload_decode_bf16", E=16, d=512, F=512, T=8, k=4, zipf_epoch=4, n_slots=4)
    router, experts = synth.gen_router(cfg), synth.gen_experts(cfg)
    layer = MoELayer(cfg, router=router, experts=experts, device=DEV, pool_slots=4, blocking=True)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for step in range(4):
        xs, x = _x(cfg, step)
        lb = torch.from_numpy(synth.zipf_logit_bias(cfg, step)).to(DEV)
        layer.forward(x, logit_bias=lb)
    e1.record()
    torch.cuda.synchronize()
    st = layer.cache.stats()
    assert st["misses"] > 0
    assert 0.0 < st["wait_ms"] <= e0.elapsed_time(e1) + 1e-3
    layer.cache.close()


@pytest.mark.parametrize("T", [1, 8])
def test_device_plan_with_shared_expert(T):
    """A Qwen1.5-MoE-shaped layer (sigmoid-gated shared expert) whose 60 routed experts live in a
    16-slot device-planned pool: the routed experts run through the pool's per-wave tables and
    the shared expert beside them; outputs equal the all-resident layer bit for bit (which runs
    the shared expert inside the routed experts' decode launches) and match the oracle."""
    cfg = synth.get_config("qwen_decode_bf16", T=T)
    router, experts = synth.gen_router(cfg), synth.gen_experts(cfg)
    shared, w_sg = synth.gen_shared(cfg), synth.gen_shared_gate(cfg)
    layer = MoELayer(cfg, router=router, experts=experts, shared=shared, w_shared_gate=w_sg, device=DEV,
                     pool_slots=16, device_plan=True)
    resident = MoELayer(cfg, router=router, experts=experts, shared=shared, w_shared_gate=w_sg, device=DEV)
    assert not layer.shared_in_decode_launch(T) and resident.shared_in_decode_launch(T)
    sim = LRUSlotCache(cfg.E, 16)
    oexp = {}
    oshared = oracle_expert(cfg, shared)
    for step in range(4):
        xs, x = _x(cfg, 20 + step)
        say(f"  case device plan + shared expert T={T} step={step}: launching")
        g = layer.forward(x)
        ref = resident.forward(x)
        torch.cuda.synchronize()
        idx = check_exact_indices(cfg, g["route"], g["perm"], T)
        sim.step(idx.ravel())
        assert torch.equal(g["out"].view(torch.int16), ref["out"].view(torch.int16)), f"step {step} differs"
        r_ref = oracle_route(cfg, xs, router, w_sg)
        for e in set(r_ref.idx.ravel().tolist()) - oexp.keys():
            oexp[e] = oracle_expert(cfg, experts[e])
        want = moe.moe_layer(decode(xs, "bf16"), r_ref, lambda e: oexp[e], cfg.E, shared=oshared)
        assert_close(to_np(g["out"]), want, "bf16")
    st = layer.cache_dev.stats()
    assert (st["hits"], st["misses"], st["evictions"], st["waves"]) == \
        (sim.stats.hits, sim.stats.misses, sim.stats.evictions, sim.stats.waves)
    assert st["misses"] > 0
    layer.cache_dev.close()
