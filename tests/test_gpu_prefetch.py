"""Cross-layer prefetch over one slot pool shared by the layers of a synthetic stack: per
layer step the cache's plans and counters equal the oracle's LRU simulation with the same
predictions, outputs equal the oracle's layer and are bit-identical to the same stack with
every expert resident, and a prefetched bundle whose copy may still be in flight is never
read early (the prediction is the layer's previous step, so hits on prefetched slots are
common)."""
import numpy as np
import pytest
import torch

from expert_offloaded_ffn_amd import synth
from expert_offloaded_ffn_amd.layer import W_CODE, MoELayer, SharedSlotPool, pack_bundles
from oracle import moe
from oracle.slot_cache import LRUSlotCache
from parity_util import assert_close, check_exact_indices, decode, oracle_expert, oracle_route, say, to_np

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _stack(L, n_slots, steps, *, prefetch, check_every=0, layer_order=False, **shape):
    base = synth.get_config("offload_decode_bf16", **shape)
    cfgs = synth.stack_configs(base, L)
    experts = synth.gen_experts(base)            # the layers share expert weights (distinct cache entries)
    bundles = pack_bundles(base, experts, base.d, base.F, pin=True)
    pool = SharedSlotPool([bundles] * L, n_slots, base.d, base.F, W_CODE["bf16"], device=DEV, layer_order=layer_order)
    routers = [synth.gen_router(c) for c in cfgs]
    layers = [MoELayer(c, router=r, experts=None, device=DEV, shared_pool=pool, layer_index=l)
              for l, (c, r) in enumerate(zip(cfgs, routers))]
    resident = [MoELayer(c, router=r, experts=experts, device=DEV) for c, r in zip(cfgs, routers)]
    E = base.E
    sim = LRUSlotCache(L * E, n_slots, n_layers=L if layer_order else 1)
    oexp = [oracle_expert(base, w) for w in experts]
    prev = [[] for _ in range(L)]
    outs = []
    for step in range(steps):
        for l in range(L):
            cfg = cfgs[l]
            xs = synth.gen_x(cfg, step)
            x = torch.from_numpy(xs.view(np.int16)).view(torch.bfloat16).to(DEV)
            lb = synth.zipf_logit_bias(cfg, step)
            nxt = (l + 1) % L
            pred = [nxt * E + e for e in prev[nxt]] if prefetch else None
            say(f"  case stack L={L} slots={n_slots} prefetch={prefetch} layer_order={layer_order} step={step} "
                f"layer={l}: launching")
            g = layers[l].forward(x, logit_bias=torch.from_numpy(lb).to(DEV), prefetch=pred)
            ref_dev = resident[l].forward(x, logit_bias=torch.from_numpy(lb).to(DEV))
            torch.cuda.synchronize()
            idx = check_exact_indices(cfg, g["route"], g["perm"], cfg.T)
            plan = sim.step((l * E + idx).ravel())
            assert g["waves"] == len(plan.waves)
            for w, wave in enumerate(plan.waves):
                assert pool.cache.wave_plan(w) == [(en.expert, en.slot, int(en.hit), en.evicted) for en in wave]
            if pred is not None:
                sim.prefetch(pred)
            st = pool.cache.stats()
            s = sim.stats
            assert (st["hits"], st["misses"], st["evictions"], st["prefetches"], st["prefetch_used"]) == \
                (s.hits, s.misses, s.evictions, s.prefetches, s.prefetch_used)
            assert st["h2d_bytes"] == (s.misses + s.prefetches) * pool.bundle_bytes
            out = to_np(g["out"])
            assert np.array_equal(out, to_np(ref_dev["out"])), "slot pool output differs from all-resident"
            outs.append(out)
            if check_every and (step * L + l) % check_every == 0:
                r_ref = oracle_route(cfg, xs, routers[l], logit_bias=lb)
                ref = moe.moe_layer(decode(xs, "bf16"), r_ref, lambda e: oexp[e], E)
                assert_close(out, ref, "bf16")
            prev[l] = sorted(set(idx.ravel().tolist()))
    pool.cache.close()
    return outs, sim


def test_stack_prefetch_plans_outputs_and_oracle():
    outs, sim = _stack(3, 16, 10, prefetch=True, check_every=4, E=16, d=256, F=256, T=3, k=4, zipf_epoch=4)
    assert sim.stats.prefetches > 0 and sim.stats.prefetch_used > 0


def test_stack_prefetch_on_and_off_agree_bitwise():
    shape = dict(E=16, d=256, F=512, T=3, k=4, zipf_epoch=3)
    a, sa = _stack(3, 14, 6, prefetch=True, **shape)
    b, sb = _stack(3, 14, 6, prefetch=False, **shape)
    assert sa.stats.prefetches > 0 and sb.stats.prefetches == 0
    for x, y in zip(a, b):
        assert np.array_equal(x, y)


def test_stack_offload_shape_few_steps():
    """The expert-offload shape (4096 x 1536 bf16 experts, 128 per layer, top-8 of 32 tokens)
    in a two-layer stack over 96 shared slots."""
    outs, sim = _stack(2, 96, 3, prefetch=True, check_every=0)
    assert sim.stats.misses > 0


def test_stack_layer_order_plans_and_outputs():
    """The layer-order victim choice on a stack that cycles through more experts than the pool
    holds: plans equal the oracle's, outputs bit-equal to all-resident, fewer bundle copies
    (misses plus prefetches) than plain LRU."""
    shape = dict(E=16, d=256, F=256, T=4, k=4, zipf_epoch=4)
    _, lo = _stack(4, 20, 8, prefetch=True, layer_order=True, check_every=7, **shape)
    _, lru = _stack(4, 20, 8, prefetch=True, **shape)
    assert lo.stats.misses + lo.stats.prefetches < lru.stats.misses + lru.stats.prefetches


def _stack_device(L, n_slots, steps, *, layer_order, freq_decay, **shape):
    base = synth.get_config("offload_decode_bf16", **shape)
    cfgs = synth.stack_configs(base, L)
    experts = synth.gen_experts(base)
    bundles = pack_bundles(base, experts, base.d, base.F, pin=True)
    pool = SharedSlotPool([bundles] * L, n_slots, base.d, base.F, W_CODE["bf16"], device=DEV,
                          layer_order=layer_order, freq_decay=freq_decay, device_plan=True)
    routers = [synth.gen_router(c) for c in cfgs]
    layers = [MoELayer(c, router=r, experts=None, device=DEV, shared_pool=pool, layer_index=l)
              for l, (c, r) in enumerate(zip(cfgs, routers))]
    resident = [MoELayer(c, router=r, experts=experts, device=DEV) for c, r in zip(cfgs, routers)]
    E = base.E
    sim = LRUSlotCache(L * E, n_slots, n_layers=L if layer_order else 1, freq_decay=freq_decay)
    for step in range(steps):
        for l in range(L):
            cfg = cfgs[l]
            xs = synth.gen_x(cfg, step)
            x = torch.from_numpy(xs.view(np.int16)).view(torch.bfloat16).to(DEV)
            lb = torch.from_numpy(synth.zipf_logit_bias(cfg, step)).to(DEV)
            say(f"  case device-planned stack L={L} slots={n_slots} layer_order={layer_order} decay={freq_decay} "
                f"step={step} layer={l}: launching")
            g = layers[l].forward(x, logit_bias=lb)
            ref = resident[l].forward(x, logit_bias=lb)
            torch.cuda.synchronize()
            idx = check_exact_indices(cfg, g["route"], g["perm"], cfg.T)
            plan = sim.step((l * E + idx).ravel())
            want_hit = np.full(L * E, -1)
            want_miss = np.full(tuple(pool.miss_slot_tables.shape), -1)
            for w, wave in enumerate(plan.waves):
                for en in wave:
                    if en.hit:
                        want_hit[en.expert] = en.slot
                    else:
                        want_miss[w, en.expert] = en.slot
            assert np.array_equal(to_np(pool.slot_table), want_hit)
            assert np.array_equal(to_np(pool.miss_slot_tables), want_miss)
            assert np.array_equal(to_np(g["out"]), to_np(ref["out"])), "device-planned stack differs from resident"
    st, s = pool.cache_dev.stats(), sim.stats
    assert (st["hits"], st["misses"], st["evictions"], st["waves"]) == (s.hits, s.misses, s.evictions, s.waves)
    pool.cache_dev.close()
    return sim


@pytest.mark.parametrize("layer_order,decay", [(True, 0.0), (True, 0.8), (False, 0.8)])
def test_stack_device_planned_policies(layer_order, decay):
    """The device planner with the layer order and / or frequency-aware victims over a shared
    pool: every layer step's tables equal the oracle's, outputs equal all-resident."""
    sim = _stack_device(4, 8, 6, layer_order=layer_order, freq_decay=decay, E=16, d=256, F=256, T=4, k=4,
                        zipf_epoch=3)
    assert sim.stats.evictions > 0 and sim.stats.waves > sim.stats.steps
