"""Parity of the HIP path (through the C ABI) with the float64 oracle on seeded inputs."""
import numpy as np
import pytest
import torch

from expert_offloaded_ffn_amd import binding as B
from expert_offloaded_ffn_amd import synth
from expert_offloaded_ffn_amd.layer import MoELayer
from oracle import moe
from parity_util import (assert_close, check_exact_indices, oracle_expert, oracle_route, route_agreement, say,
                         to_np, decode)

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _build(cfg, *, pool_slots=None, blocking=False):
    router = synth.gen_router(cfg)
    experts = synth.gen_experts(cfg)
    shared = synth.gen_shared(cfg) if cfg.F_shared else None
    w_sg = synth.gen_shared_gate(cfg) if cfg.shared_gate else None
    sb = synth.gen_select_bias(cfg) if cfg.select_bias else None
    layer = MoELayer(cfg, router=router, experts=experts, shared=shared, w_shared_gate=w_sg, select_bias=sb,
                     device=DEV, pool_slots=pool_slots, blocking=blocking)
    return layer, dict(router=router, experts=experts, shared=shared, w_sg=w_sg, sb=sb)


def _x_dev(cfg, x_store):
    if cfg.act_dtype == "f32":
        return torch.from_numpy(x_store).to(DEV)
    return torch.from_numpy(x_store.view(np.int16)).view(torch.bfloat16).to(DEV)


def cover_tokens(g, k, block=64, extra=0, seed=0):
    """Tokens whose rows cover every expert's rows in blocks of `block` grouped rows: for every
    expert, the token of its first row, of every block's last row and of its last row (so
    every m-tile of any height that is a multiple of `block`, including a nearly empty last
    one, has a checked row), plus `extra` random tokens. Read off the device's grouping."""
    off = to_np(g["perm"]["offsets"]).astype(np.int64)
    src = to_np(g["perm"]["perm_src"]).astype(np.int64)
    rows = []
    for e in range(len(off) - 1):
        lo, hi = int(off[e]), int(off[e + 1])
        if hi > lo:
            rows += [lo, hi - 1] + list(range(lo + block - 1, hi, block))
    toks = set((src[np.array(rows)] // k).tolist())
    if extra:
        T = len(src) // k
        rng = np.random.default_rng(seed)
        toks |= set(rng.choice(T, min(extra, T), replace=False).tolist())
    return np.array(sorted(toks))


def _run_and_check(cfg, layer, w, T, xi=0, tokens=None, logit_bias=None, tokens_fn=None):
    """tokens: the tokens checked against the oracle (all when None); tokens_fn(g) picks them
    from the device's routing instead."""
    x_store = synth.gen_x(cfg, xi, T=T)
    x = _x_dev(cfg, x_store)
    lb = None if logit_bias is None else torch.from_numpy(logit_bias).to(DEV)
    say(f"  case {cfg.name} T={T} x={xi}: launching")
    g = layer.forward(x, logit_bias=lb)
    torch.cuda.synchronize()
    say("    done")
    check_exact_indices(cfg, g["route"], g["perm"], T)
    r_ref = oracle_route(cfg, x_store, w["router"], w["w_sg"], w["sb"], logit_bias)
    same = route_agreement(cfg, r_ref, g["route"], key_tol=1e-4)
    if cfg.shared_gate:
        err = np.abs(to_np(g["route"]["shared_gate"]) - r_ref.shared_gate).max()
        assert err <= 1e-4, f"shared gate err {err}"
    if tokens_fn is not None:
        tokens = tokens_fn(g)
    toks = np.arange(T) if tokens is None else np.asarray(tokens)
    toks = toks[same[toks]]
    if tokens is not None:
        say(f"    checking {len(toks)} of {T} tokens")
    cache = {}

    def expert(e):
        if e not in cache:
            cache.clear()
            cache[e] = oracle_expert(cfg, w["experts"][e])
        return cache[e]

    shared = oracle_expert(cfg, w["shared"]) if w["shared"] is not None else None
    ref = moe.moe_layer(decode(x_store, cfg.act_dtype), r_ref, expert, cfg.E, shared=shared,
                        quant_act=cfg.dtype == "fp8", tokens=toks)
    got = to_np(g["out"])[toks]
    assert_close(got, ref, cfg.dtype)
    return g


def test_tiny_fp32_layer():
    cfg = synth.get_config("tiny_fp32")
    layer, w = _build(cfg)
    for xi in range(3):
        _run_and_check(cfg, layer, w, cfg.T, xi)


@pytest.mark.parametrize("T,d,E,k,F", [(333, 512, 8, 2, 1024), (97, 256, 60, 4, 384), (1, 256, 16, 4, 128),
                                       (700, 256, 32, 8, 256)])
def test_bf16_layer_reduced(T, d, E, k, F):
    cfg = synth.get_config("mixtral_prefill_bf16", T=T, d=d, E=E, k=k, F=F, name=f"bf16_T{T}_d{d}_E{E}_k{k}_F{F}")
    layer, w = _build(cfg)
    _run_and_check(cfg, layer, w, T)


@pytest.mark.parametrize("T", [256, 257, 300, 320, 321, 1088, 1089])
def test_bf16_last_tile_sizes(T):
    """E=2, k=2: both experts get all T rows. Around 256 + 64 rows an expert's last m-tile
    switches between one tile of up to 320 rows and an extra tile; every row is checked."""
    cfg = synth.get_config("mixtral_prefill_bf16", T=T, d=256, E=2, k=2, F=512, name=f"lasttile_T{T}")
    layer, w = _build(cfg)
    g = _run_and_check(cfg, layer, w, T)
    assert to_np(g["route"]["counts"]).tolist() == [T, T]


@pytest.mark.parametrize("T,d,E,k,F", [(200, 256, 16, 1, 256), (130, 256, 96, 6, 256)])
def test_bf16_layer_top1_and_many_experts(T, d, E, k, F):
    """top-1 routing (gates are 1 after renormalisation), and more experts than one 64-lane group."""
    cfg = synth.get_config("mixtral_prefill_bf16", T=T, d=d, E=E, k=k, F=F, name=f"bf16b_T{T}_E{E}_k{k}")
    layer, w = _build(cfg)
    g = _run_and_check(cfg, layer, w, T)
    if k == 1:
        np.testing.assert_allclose(to_np(g["route"]["gate"]), 1.0, rtol=0, atol=1e-6)


@pytest.mark.parametrize("config_name", ["mixtral_prefill_bf16", "qwen_decode_bf16", "dsv3_prefill_fp8"])
def test_empty_batch(config_name):
    """T = 0 runs through every call of the layer and returns an empty output."""
    overrides = {"d": 256, "F": 256} if config_name == "mixtral_prefill_bf16" else {}
    if config_name == "dsv3_prefill_fp8":
        overrides = dict(d=512, E=32, k=8, F=256, F_shared=256, n_groups=8, topk_groups=4)
    if config_name == "qwen_decode_bf16":
        overrides = dict(T=1)
    cfg = synth.get_config(config_name, name=f"empty_{config_name}", **overrides)
    layer, _ = _build(cfg)
    x = torch.empty(0, cfg.d, device=DEV, dtype=torch.float32 if cfg.act_dtype == "f32" else torch.bfloat16)
    say(f"  case empty batch {config_name}: launching")
    g = layer.forward(x)
    torch.cuda.synchronize()
    assert tuple(g["out"].shape) == (0, cfg.d)
    assert to_np(g["perm"]["offsets"]).tolist() == [0] * (cfg.E + 1)


def test_mixtral_full_size_sampled():
    """The full Mixtral-shaped layer: every expert's rows checked in blocks of 64 (each of its
    m-tiles, the taller last one included), plus random tokens to at least 256."""
    cfg = synth.get_config("mixtral_prefill_bf16")
    layer, w = _build(cfg)
    _run_and_check(cfg, layer, w, cfg.T, 0, tokens_fn=lambda g: cover_tokens(g, cfg.k, 64, extra=160))


@pytest.mark.parametrize("T", [1, 8, 64])
def test_qwen_decode_full_size(T):
    cfg = synth.get_config("qwen_decode_bf16", T=T)
    layer, w = _build(cfg)
    for xi in range(2):
        _run_and_check(cfg, layer, w, T, xi)


def test_determinism_bitwise():
    cfg = synth.get_config("mixtral_prefill_bf16", T=600, d=512, F=1024, name="det")
    layer, _ = _build(cfg)
    x = _x_dev(cfg, synth.gen_x(cfg, 0))
    a = layer.forward(x)["out"].clone()
    b = layer.forward(x)["out"].clone()
    torch.cuda.synchronize()
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))


def test_skewed_routing_and_empty_experts():
    """A large logit prior sends every token to experts 3 and 5 (others get no rows)."""
    cfg = synth.get_config("mixtral_prefill_bf16", T=300, d=256, F=256, name="skew")
    layer, w = _build(cfg)
    lb = np.zeros(cfg.E, np.float32)
    lb[3], lb[5] = 40.0, 30.0
    g = _run_and_check(cfg, layer, w, cfg.T, 0, logit_bias=lb)
    counts = to_np(g["route"]["counts"])
    assert counts[3] == cfg.T and counts[5] == cfg.T and counts.sum() == 2 * cfg.T


def test_permute_gather_and_e4m3_quantisation_bit_exact():
    from oracle import formats
    cfg = synth.get_config("dsv3_prefill_fp8", T=200, d=512, E=32, k=8, n_groups=8, topk_groups=4)
    rng = np.random.default_rng(5)
    idx = np.stack([rng.choice(cfg.E, cfg.k, replace=False) for _ in range(cfg.T)]).astype(np.int32)
    x_store = synth.gen_x(cfg, 0)
    x = _x_dev(cfg, x_store)
    say("  case permute gather/quant: launching")
    p = B.permute(torch.from_numpy(idx).to(DEV), cfg.E, x=x, out_dtype=B.MOE_FP8_E4M3, gather=1)
    q = B.permute(torch.from_numpy(idx).to(DEV), cfg.E, x=x, out_dtype=B.MOE_FP8_E4M3, gather=0)
    c = B.permute(torch.from_numpy(idx).to(DEV), cfg.E, x=x, gather=1)
    torch.cuda.synchronize()
    off, src, dst = moe.permutation(idx, cfg.E)
    assert np.array_equal(to_np(p["perm_src"]), src)
    xf = decode(x_store, "bf16")
    codes, scales = formats.quantize_rows_e4m3(xf)
    assert np.array_equal(to_np(q["x_out"]), codes)
    assert np.array_equal(to_np(q["x_out_scale"]), scales)
    assert np.array_equal(to_np(p["x_out"]), codes[src // cfg.k])
    assert np.array_equal(to_np(p["x_out_scale"]), scales[src // cfg.k])
    assert np.array_equal(to_np(c["x_out"]), xf[src // cfg.k])


def _rounding_case_values():
    """Every e4m3 code value, every midpoint between consecutive codes and the two bf16 neighbours
    of each midpoint, both signs: the exact ties and near-ties that random inputs almost never
    reach. All of them are bf16 values."""
    from oracle import formats
    pos = formats.e4m3_table()[:0x7F]
    mids = (pos[:-1] + pos[1:]) / 2
    mb = synth.to_bf16_bits(mids.astype(np.float32)).astype(np.int64)
    below = formats.decode_bf16((mb - 1).astype(np.uint16))
    above = formats.decode_bf16((mb + 1).astype(np.uint16))
    v = np.concatenate([pos, mids, below, above])
    v = np.concatenate([v, -v])
    assert np.array_equal(formats.decode_bf16(synth.to_bf16_bits(v.astype(np.float32))), v)
    return v


def _rounding_case_rows(v, block, ks):
    """One row per power of two 2^k in ks: blocks of `block` columns, each led by 448 * 2^k (so the
    block's e4m3 scale, or MX exponent, is exactly 2^k) and followed by values of v times 2^k."""
    per = block - 1
    nb = -(-len(v) // per)
    rows = []
    for k in ks:
        r = np.zeros((nb, block))
        r[:, 0] = 448.0 * 2.0 ** k
        vv = np.zeros(nb * per)
        vv[:len(v)] = v * 2.0 ** k
        r[:, 1:] = vv.reshape(nb, per)
        rows.append(r.reshape(-1))
    return np.stack(rows)


def test_e4m3_and_mxfp8_rounding_at_ties_bit_exact():
    """The device's e4m3 rounding (a gfx950 conversion instruction) at every code, every midpoint
    between codes and the bf16 neighbours of each midpoint, through moe_permute's e4m3 (per 128
    columns) and MXFP8 (per 32) token quantisation: codes and scales bit for bit against the oracle,
    with block scales 2^k exact so each test value reaches the rounding unchanged."""
    from oracle import formats
    v = _rounding_case_values()
    for block, out in ((128, B.MOE_FP8_E4M3), (32, B.MOE_MXFP8)):
        xf = _rounding_case_rows(v, block, (0, -5, 3))
        bits = synth.to_bf16_bits(xf.astype(np.float32))
        x = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(DEV)
        T = x.shape[0]
        idx = torch.zeros(T, 1, dtype=torch.int32, device=DEV)
        say(f"  case rounding ties, {block}-column blocks: launching")
        q = B.permute(idx, 1, x=x, out_dtype=out, gather=0)
        torch.cuda.synchronize()
        if out == B.MOE_FP8_E4M3:
            codes, scales = formats.quantize_rows_e4m3(xf)
            assert np.array_equal(to_np(q["x_out_scale"]), scales)
        else:
            codes, scales = formats.quantize_rows_mxfp8(xf)
            assert np.array_equal(to_np(q["x_out_scale"]), scales)
        got = to_np(q["x_out"])
        bad = np.argwhere(got != codes)
        assert bad.size == 0, f"{len(bad)} codes differ, first at {bad[0]}: value {xf[tuple(bad[0])]}, got " \
                              f"{got[tuple(bad[0])]:#04x}, oracle {codes[tuple(bad[0])]:#04x}"


def test_dsv3_routing_full_size():
    """Group-limited sigmoid routing with selection bias at the full DeepSeek-V3 shape (bf16 router)."""
    cfg = synth.get_config("dsv3_prefill_fp8")
    router = synth.gen_router(cfg)
    sb = synth.gen_select_bias(cfg)
    x_store = synth.gen_x(cfg, 0)
    x = _x_dev(cfg, x_store)
    wr = torch.from_numpy(np.ascontiguousarray(router.T).view(np.int16)).view(torch.bfloat16).to(DEV)
    say("  case dsv3 route full: launching")
    r = B.route(x, wr, k=cfg.k, score_fn=B.MOE_SIGMOID, route_scale=cfg.route_scale, n_groups=8, topk_groups=4,
                group_topn=2, select_bias=torch.from_numpy(sb).to(DEV))
    p = B.permute(r["idx"], cfg.E)
    torch.cuda.synchronize()
    check_exact_indices(cfg, r, p, cfg.T)
    r_ref = oracle_route(cfg, x_store, router, select_bias=sb)
    same = route_agreement(cfg, r_ref, r, key_tol=1e-5)
    say(f"    near-tie mismatches: {int((~same).sum())} of {cfg.T}")
    g = to_np(r["gate"])
    np.testing.assert_allclose(g.sum(axis=1), 2.5, rtol=1e-5)


_WIDE_CASES = [
    # moe_route's large-batch logits (more than 256 tokens over more than 64 columns, d a multiple
    # of 64: 64-token x 128-column tiles over all of K through a 6-stage LDS ring): ragged token
    # and column tiles, K of 3, 5, 1 and 12 stages, the shared-gate column inside a partly filled
    # column tile
    ("dsv3_prefill_fp8", dict(T=300, d=192)),
    ("qwen_decode_bf16", dict(T=600, E=100, d=320)),
    ("mixtral_prefill_bf16", dict(T=257, E=72, d=64)),
    ("qwen_decode_bf16", dict(T=1000, E=130, d=768)),
    # d a multiple of 32 but not of 64: the same batches fall back to route_logits_mfma's 64-token
    # x 64-column blocks with K split over four waves
    ("qwen_decode_bf16", dict(T=300, E=100, d=224)),
]


@pytest.mark.parametrize("name,over", _WIDE_CASES)
def test_route_logits_wide_tiles(name, over):
    cfg = synth.get_config(name, **over)
    router = synth.gen_router(cfg)
    w_sg = synth.gen_shared_gate(cfg) if cfg.shared_gate else None
    sb = synth.gen_select_bias(cfg) if cfg.select_bias else None
    x_store = synth.gen_x(cfg, 0)
    x = _x_dev(cfg, x_store)
    wr = torch.from_numpy(np.ascontiguousarray(router.T).view(np.int16)).view(torch.bfloat16).to(DEV)
    sg_dev = None if w_sg is None else torch.from_numpy(w_sg.view(np.int16)).view(torch.bfloat16).to(DEV)
    say(f"  case route wide {name} {over}: launching")
    r = B.route(x, wr, k=cfg.k, score_fn=B.MOE_SIGMOID if cfg.score_fn == "sigmoid" else B.MOE_SOFTMAX,
                renormalize=cfg.renormalize, route_scale=cfg.route_scale, n_groups=cfg.n_groups,
                topk_groups=cfg.topk_groups, group_topn=cfg.group_topn,
                select_bias=None if sb is None else torch.from_numpy(sb).to(DEV), w_shared_gate=sg_dev)
    p = B.permute(r["idx"], cfg.E)
    torch.cuda.synchronize()
    say("    done")
    check_exact_indices(cfg, r, p, cfg.T)
    r_ref = oracle_route(cfg, x_store, router, w_sg, sb)
    route_agreement(cfg, r_ref, r, key_tol=1e-5)
    if cfg.shared_gate:
        err = np.abs(to_np(r["shared_gate"]) - r_ref.shared_gate).max()
        assert err <= 1e-5, f"shared gate err {err}"


@pytest.mark.parametrize("T,d,E,k,F,Fs,G,TG", [(300, 512, 16, 4, 256, 256, 4, 2), (70, 256, 32, 8, 128, 128, 8, 4)])
def test_fp8_layer_reduced(T, d, E, k, F, Fs, G, TG):
    cfg = synth.get_config("dsv3_prefill_fp8", T=T, d=d, E=E, k=k, F=F, F_shared=Fs, n_groups=G, topk_groups=TG,
                           name=f"fp8_T{T}_d{d}_E{E}_k{k}_F{F}")
    layer, w = _build(cfg)
    _run_and_check(cfg, layer, w, T)


def test_dsv3_fp8_full_size_sampled():
    """The full DeepSeek-V3-shaped layer: for every one of the 256 experts its first and last row
    and the last row of every block of 64 of its rows are checked (so each m-tile, including a
    nearly empty last one, has checked rows), with the shared expert on every checked token."""
    cfg = synth.get_config("dsv3_prefill_fp8")
    layer, w = _build(cfg)
    _run_and_check(cfg, layer, w, cfg.T, 0, tokens_fn=lambda g: cover_tokens(g, cfg.k, 64))


def test_fp8_layer_many_tiles_every_row():
    """More gate/up tiles (about 512) and down tiles than the persistent grid has blocks, so every
    block takes several tiles through the same LDS ring and the per-XCD queues hand tiles across
    XCDs; every row of the layer is checked."""
    cfg = synth.get_config("dsv3_prefill_fp8", T=2048, d=512, E=64, k=8, F=512, F_shared=512, n_groups=8,
                           topk_groups=4, name="fp8_many_tiles")
    layer, w = _build(cfg)
    g = _run_and_check(cfg, layer, w, cfg.T)
    assert to_np(g["route"]["counts"]).max() > 256


@pytest.mark.parametrize("T", [1, 8])
def test_decode_graph_replay_matches_eager(T):
    """The whole decode layer captured as one HIP graph: every replay (with eager work and
    synchronisations in between) equals the eager result bit for bit, for changing inputs."""
    cfg = synth.get_config("qwen_decode_bf16", T=T)
    layer, w = _build(cfg)
    x_static = _x_dev(cfg, synth.gen_x(cfg, 0))
    say(f"  case decode graph T={T}: capture")
    graph, outs = layer.capture(x_static)
    for i in range(4):
        xi = _x_dev(cfg, synth.gen_x(cfg, 10 + i))
        x_static.copy_(xi)
        graph.replay()
        torch.cuda.synchronize()
        got = outs["out"].clone()
        ref = layer.forward(xi)["out"]            # eager work between replays
        torch.cuda.synchronize()
        assert torch.equal(got.view(torch.int16), ref.view(torch.int16)), f"replay {i} differs from eager"
    # and the replayed output still matches the oracle
    _run_and_check(cfg, layer, w, T, 13)


_RP_CASES = [
    # config, overrides, T: the sliced-logits paths (T <= 16 and 17..64, E <= 256, bf16) and the
    # two-call path
    ("qwen_decode_bf16", {}, 1),
    ("qwen_decode_bf16", {}, 8),
    ("qwen_decode_bf16", {}, 17),
    ("qwen_decode_bf16", {}, 64),
    ("qwen_decode_bf16", {}, 65),                                         # two calls
    ("qwen_decode_bf16", {}, 16),
    ("dsv3_prefill_fp8", dict(d=512, E=256, k=8), 16),                  # grouped sigmoid, E = 256
    ("dsv3_prefill_fp8", dict(d=256, E=64, k=8, n_groups=8, topk_groups=3), 5),
    ("offload_decode_bf16", dict(d=512), 7),                              # E = 128, logit prior
    ("offload_decode_bf16", {}, 12),                                      # d = 4096
    ("offload_decode_bf16", {}, 32),                                      # d = 4096, 17..64 tokens
    ("mixtral_prefill_bf16", dict(d=96, k=1), 3),                         # a partial K slice, top-1
    ("mixtral_prefill_bf16", dict(d=256, E=40, k=12), 9),                 # k > 8
    ("dsv3_prefill_fp8", dict(d=512, E=256, k=8), 40),                  # grouped sigmoid, 17..64 tokens
    ("mixtral_prefill_bf16", dict(d=256), 200),                           # two calls
]


@pytest.mark.parametrize("name,over,T", _RP_CASES)
def test_route_permute_against_route_then_permute(name, over, T):
    """moe_route_permute meets the routing contract against the oracle. Where it makes the two
    calls it equals moe_route followed by moe_permute bit for bit; on the sliced-logits path its
    keys (summed over K slices in another order) agree with theirs to rounding."""
    cfg = synth.get_config(name, T=T, **over)
    router = synth.gen_router(cfg)
    w_sg = synth.gen_shared_gate(cfg) if cfg.shared_gate else None
    sb = synth.gen_select_bias(cfg) if cfg.select_bias else None
    lb = np.random.default_rng([7, T]).normal(0, 2.0, cfg.E).astype(np.float32) if name.startswith("offload") else None
    x_store = synth.gen_x(cfg, 0, T=T)
    x = _x_dev(cfg, x_store)
    wr = torch.from_numpy(np.ascontiguousarray(router.T).view(np.int16)).view(torch.bfloat16).to(DEV)
    sg_dev = None if w_sg is None else torch.from_numpy(w_sg.view(np.int16)).view(torch.bfloat16).to(DEV)
    kw = dict(k=cfg.k, score_fn=B.MOE_SIGMOID if cfg.score_fn == "sigmoid" else B.MOE_SOFTMAX,
              renormalize=cfg.renormalize, route_scale=cfg.route_scale, n_groups=cfg.n_groups,
              topk_groups=cfg.topk_groups, group_topn=cfg.group_topn,
              logit_bias=None if lb is None else torch.from_numpy(lb).to(DEV),
              select_bias=None if sb is None else torch.from_numpy(sb).to(DEV), w_shared_gate=sg_dev)
    say(f"  case route_permute {name} {over} T={T}: launching")
    fused = B.route_permute(x, wr, **kw)
    r = B.route(x, wr, **kw)
    p = B.permute(r["idx"], cfg.E)
    torch.cuda.synchronize()
    say("    done")
    check_exact_indices(cfg, fused, fused, T)
    r_ref = oracle_route(cfg, x_store, router, w_sg, sb, lb)
    route_agreement(cfg, r_ref, fused, key_tol=1e-4)
    sliced = T <= 64 and cfg.E <= 256
    if not sliced:
        for key, ref in [("scores", r), ("idx", r), ("gate", r), ("counts", r), ("shared_gate", r),
                         ("offsets", p), ("perm_src", p), ("perm_dst", p)]:
            if ref[key] is None:
                assert fused[key] is None
                continue
            a, b = fused[key].cpu(), ref[key].cpu()
            assert torch.equal(a.view(torch.int32) if a.dtype == torch.float32 else a,
                               b.view(torch.int32) if b.dtype == torch.float32 else b), f"{key} differs"
        return
    kf, ks = to_np(fused["scores"]), to_np(r["scores"])
    assert np.abs(kf - ks).max() <= 1e-5 * max(1.0, np.abs(ks).max())
    if cfg.shared_gate:
        assert np.abs(to_np(fused["shared_gate"]) - to_np(r["shared_gate"])).max() <= 1e-6


def test_route_permute_empty_batch():
    cfg = synth.get_config("qwen_decode_bf16", T=0)
    wr = torch.zeros(cfg.E, cfg.d, device=DEV, dtype=torch.bfloat16)
    x = torch.zeros(0, cfg.d, device=DEV, dtype=torch.bfloat16)
    out = B.route_permute(x, wr, k=cfg.k)
    torch.cuda.synchronize()
    assert out["offsets"].cpu().eq(0).all()


@pytest.mark.parametrize("T,Fs", [(1, 512), (5, 512), (64, 512), (100, 512), (1, 5632), (3, 5632), (7, 5632),
                                  (64, 5632), (100, 5632)])
def test_grouped_ffn_batch_equals_separate_calls(T, Fs):
    """The shared and the routed experts through moe_grouped_ffn_batch (one launch per GEMM for a
    decode step, else one call after the other) give exactly the outputs of two moe_grouped_ffn calls.
    With F_shared = 5632 and at most 4 rows the shared expert's down projection is split over K
    across workgroups (fp32 partials added by the last to arrive); repeating the calls over a
    workspace filled with stale bytes checks that the arrival counts start from zero every time."""
    cfg = synth.get_config("qwen_decode_bf16", T=T, d=256, E=16, k=4, F=256, F_shared=Fs)
    layer, w = _build(cfg)
    x = _x_dev(cfg, synth.gen_x(cfg, 0, T=T))
    say(f"  case grouped_ffn_batch T={T}: launching")
    r = B.route_permute(x, layer.w_router_t, w_shared_gate=layer.w_sg, **layer.route_args())
    rows = T * cfg.k
    offs = torch.tensor([0, T], dtype=torch.int32).to(DEV)
    y_sep = B.grouped_ffn(layer.table, rows, r["offsets"], x, a_row_src=r["perm_src"], a_row_div=cfg.k)
    s_sep = B.grouped_ffn(layer.shared.table, T, offs, x)
    probs = [B.ffn_problem(layer.shared.table, T, offs, x),
             B.ffn_problem(layer.table, rows, r["offsets"], x, a_row_src=r["perm_src"], a_row_div=cfg.k)]
    ws = torch.empty(B.grouped_ffn_batch_workspace_size(probs), device=DEV, dtype=torch.uint8)
    s_bat, y_bat = B.grouped_ffn_batch(probs, ws=ws)
    torch.cuda.synchronize()
    s_first, y_first = s_bat.clone(), y_bat.clone()
    ws.fill_(0x5A)   # stale bytes everywhere, arrival counts included
    for _ in range(2):
        s_bat, y_bat = B.grouped_ffn_batch(probs, ws=ws)
        s_sep2 = B.grouped_ffn(layer.shared.table, T, offs, x)
    torch.cuda.synchronize()
    say("    done")
    assert torch.equal(y_bat.view(torch.int16).cpu(), y_sep.view(torch.int16).cpu())
    assert torch.equal(s_bat.view(torch.int16).cpu(), s_sep.view(torch.int16).cpu())
    assert torch.equal(s_first.view(torch.int16).cpu(), s_sep.view(torch.int16).cpu())
    assert torch.equal(y_first.view(torch.int16).cpu(), y_sep.view(torch.int16).cpu())
    assert torch.equal(s_sep2.view(torch.int16).cpu(), s_sep.view(torch.int16).cpu())
    # and the shared expert's output against the oracle
    shared = oracle_expert(cfg, w["shared"])
    ref = moe.swiglu_ffn(decode(synth.gen_x(cfg, 0, T=T), cfg.act_dtype), shared.w_gate, shared.w_up, shared.w_down)
    assert_close(to_np(s_bat), ref, cfg.dtype, "shared expert")


def test_grouped_ffn_batch_split_beside_wide_routed():
    """A batch whose first problem splits its down projection over K (2 rows of the 5632-wide
    shared expert) beside a routed problem of another batch with more than 16 rows per expert:
    the shared launch then covers the routed experts in several 16-row passes, and both outputs
    must equal those of separate calls bit for bit."""
    cfg = synth.get_config("qwen_decode_bf16", T=2, d=256, E=4, k=2, F=256, F_shared=5632)
    layer, w = _build(cfg)
    T2 = 48
    x1 = _x_dev(cfg, synth.gen_x(cfg, 0, T=2))
    x2 = _x_dev(cfg, synth.gen_x(cfg, 1, T=T2))
    say("  case grouped_ffn_batch split + 48-token routed: launching")
    r = B.route_permute(x2, layer.w_router_t, w_shared_gate=layer.w_sg, **layer.route_args())
    counts = r["offsets"].cpu().diff()
    assert int(counts.max()) > 16
    rows = T2 * cfg.k
    offs = torch.tensor([0, 2], dtype=torch.int32).to(DEV)
    y_sep = B.grouped_ffn(layer.table, rows, r["offsets"], x2, a_row_src=r["perm_src"], a_row_div=cfg.k)
    s_sep = B.grouped_ffn(layer.shared.table, 2, offs, x1)
    probs = [B.ffn_problem(layer.shared.table, 2, offs, x1),
             B.ffn_problem(layer.table, rows, r["offsets"], x2, a_row_src=r["perm_src"], a_row_div=cfg.k)]
    ws = torch.empty(B.grouped_ffn_batch_workspace_size(probs), device=DEV, dtype=torch.uint8)
    ws.fill_(0x5A)
    s_bat, y_bat = B.grouped_ffn_batch(probs, ws=ws)
    torch.cuda.synchronize()
    say("    done")
    assert torch.equal(y_bat.view(torch.int16).cpu(), y_sep.view(torch.int16).cpu())
    assert torch.equal(s_bat.view(torch.int16).cpu(), s_sep.view(torch.int16).cpu())
    shared = oracle_expert(cfg, w["shared"])
    ref = moe.swiglu_ffn(decode(synth.gen_x(cfg, 0, T=2), cfg.act_dtype), shared.w_gate, shared.w_up, shared.w_down)
    assert_close(to_np(s_bat), ref, cfg.dtype, "shared expert")


@pytest.mark.parametrize("T", [64, 300])
def test_max_experts_and_top_k(T):
    """The largest routing the ABI takes: 1024 experts, top-32. T = 64 takes the decode kernels
    (at most 64 rows per expert), T = 300 the prefill tile map over 1024 experts."""
    cfg = synth.get_config("mixtral_prefill_bf16", T=T, d=256, F=256, E=1024, k=32, name="maxE")
    layer, w = _build(cfg)
    _run_and_check(cfg, layer, w, T, 0)


def test_grouped_routing_at_64_groups():
    """Group-limited sigmoid routing with selection bias at 1024 experts in 64 groups (8 kept,
    top-2 sum per group), top-16, against the oracle's routing contract."""
    cfg = synth.get_config("dsv3_prefill_fp8", T=200, d=256, E=1024, k=16, n_groups=64, topk_groups=8,
                           group_topn=2)
    router = synth.gen_router(cfg)
    sb = synth.gen_select_bias(cfg)
    x_store = synth.gen_x(cfg, 0, T=cfg.T)
    x = _x_dev(cfg, x_store)
    wr = torch.from_numpy(np.ascontiguousarray(router.T).view(np.int16)).view(torch.bfloat16).to(DEV)
    say("  case grouped routing 1024 experts / 64 groups: launching")
    r = B.route(x, wr, k=cfg.k, score_fn=B.MOE_SIGMOID, route_scale=cfg.route_scale, n_groups=64, topk_groups=8,
                group_topn=2, select_bias=torch.from_numpy(sb).to(DEV))
    p = B.permute(r["idx"], cfg.E)
    torch.cuda.synchronize()
    say("    done")
    check_exact_indices(cfg, r, p, cfg.T)
    r_ref = oracle_route(cfg, x_store, router, select_bias=sb)
    route_agreement(cfg, r_ref, r, key_tol=1e-5)


@pytest.mark.parametrize("name,over", [("mixtral_prefill_bf16", dict(T=1200, d=256, F=512)),
                                       ("dsv3_prefill_fp8", dict(T=400, d=512, E=32, k=8, F=256, F_shared=256,
                                                                 n_groups=8, topk_groups=4))])
def test_prefill_under_zipf_skew(name, over):
    """Prefill with a Zipf(1.1) log-prior on the routing logits: a few experts get several times
    the average rows (many m-tiles), others few; the grouped GEMMs stay within tolerance."""
    import dataclasses
    cfg = synth.get_config(name, **over)
    layer, w = _build(cfg)
    lb = synth.zipf_logit_bias(dataclasses.replace(cfg, zipf_alpha=1.1, zipf_epoch=1), 0)
    g = _run_and_check(cfg, layer, w, cfg.T, 0, tokens=np.arange(0, cfg.T, 3), logit_bias=lb)
    counts = to_np(g["route"]["counts"])
    assert counts.max() >= 2 * counts.mean()   # the skew is real


@pytest.mark.parametrize("T", [1, 2, 3])
def test_decode_routed_down_split(T):
    """A Mixtral-shaped expert (F = 14336) serving 1-3 tokens: the routed problem has at most 4
    rows, so its down projection is split over K across 8 workgroups per 32-column group, and
    the last to arrive adds the partials (T = 3 has 6 rows and is not split)."""
    cfg = synth.get_config("mixtral_prefill_bf16", T=T, d=256, name="decode_split")
    layer, w = _build(cfg)
    for xi in range(2):
        _run_and_check(cfg, layer, w, T, xi)
