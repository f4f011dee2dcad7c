"""The seeded input generators: determinism, storage formats, the Zipf prior."""
import numpy as np
import torch

from expert_offloaded_ffn_amd import synth
from oracle import formats


def test_bf16_rounding_matches_torch():
    rng = np.random.default_rng(0)
    x = (rng.standard_normal(100000) * 10).astype(np.float32)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(synth.to_bf16_bits(x), ref)


def test_generation_is_deterministic_and_per_tensor():
    cfg = synth.get_config("tiny_fp32")
    a = synth.gen_expert(cfg, 3)
    b = synth.gen_experts(cfg)[3]
    for u, v in zip(a, b):
        assert np.array_equal(u, v)
    assert not np.array_equal(synth.gen_expert(cfg, 2)[0], a[0])
    assert np.array_equal(synth.gen_x(cfg, 1), synth.gen_x(cfg, 1))
    assert not np.array_equal(synth.gen_x(cfg, 1), synth.gen_x(cfg, 2))


def test_weight_statistics():
    cfg = synth.get_config("qwen_decode_bf16")
    wg, wu, wd = synth.gen_expert(cfg, 0)
    g = formats.decode_bf16(wg)
    d = formats.decode_bf16(wd)
    assert wg.shape == (2048, 1408) and wd.shape == (1408, 2048)
    assert abs(g.std() * np.sqrt(2048) - 1) < 0.01
    assert abs(d.std() * np.sqrt(1408) - 1) < 0.01
    x = formats.decode_bf16(synth.gen_x(cfg, 0, T=64))
    assert abs(x.std() - 1) < 0.02


def test_fp8_weight_blocks():
    cfg = synth.get_config("dsv3_prefill_fp8", E=1, F=256, d=384)
    (gq, gs), (uq, us), (dq, ds) = synth.gen_expert(cfg, 0)
    assert gq.dtype == np.uint8 and gq.shape == (384, 256) and gs.shape == (3, 2)
    assert dq.shape == (256, 384) and ds.shape == (2, 3)
    w = formats.dequantize_weight_blocks(gq, gs)
    # each block's max magnitude is exactly its scale * 448
    blk = np.abs(w).reshape(3, 128, 2, 128).max(axis=(1, 3))
    np.testing.assert_allclose(blk, gs.astype(np.float64) * 448.0, rtol=1e-6)


def test_zipf_prior():
    cfg = synth.get_config("offload_decode_bf16")
    b0 = synth.zipf_logit_bias(cfg, 0)
    assert np.array_equal(b0, synth.zipf_logit_bias(cfg, 63))
    assert not np.array_equal(b0, synth.zipf_logit_bias(cfg, 64))
    p = np.exp(b0.astype(np.float64))
    assert abs(p.sum() - 1.0) < 1e-5
    ranks = np.sort(p)[::-1]
    np.testing.assert_allclose(ranks[0] / ranks[1], 2.0 ** 1.1, rtol=1e-5)
    flat = synth.zipf_logit_bias(synth.get_config("offload_decode_bf16", zipf_alpha=0.0), 0)
    np.testing.assert_allclose(flat, -np.log(128.0), rtol=1e-6)
