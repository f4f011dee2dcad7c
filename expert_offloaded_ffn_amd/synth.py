"""Seeded synthetic inputs for one Mixture-of-Experts FFN layer.

This module only draws random tensors and stores them in the formats the layer
consumes (fp32, bf16 bit patterns, OCP e4m3 codes with fp32 block scales, OCP MXFP4
codes with E8M0 scales per 32 inputs). It
holds none of the layer's arithmetic: routing, grouping, the expert FFN and the
combine live in the HIP library and, independently, in the CPU oracle. Both
sides read the exact bytes produced here.

Workloads (shapes and dtypes of well-known MoE layers; the pages discuss
Mixtral, Qwen-MoE and DeepSeek-family models without fixing their shapes):

* ``tiny_fp32``            T=16, d=128, E=8, top-2 softmax, SwiGLU F=256, fp32.
* ``mixtral_prefill_bf16`` T=4096, d=4096, E=8, top-2 softmax, F=14336, bf16.
* ``qwen_decode_bf16``     d=2048, E=60, top-4 softmax, F=1408, one shared
                           expert F=5632 behind a sigmoid scalar gate,
                           T in {1, 8, 64}, bf16.
* ``dsv3_prefill_fp8``     T=8192, d=7168, E=256, top-8 sigmoid + per-expert
                           selection bias, 8 groups / keep 4 / group score =
                           sum of top-2, gates renormalised and scaled by 2.5,
                           F=2048 plus one shared expert F=2048; e4m3 weights
                           with per-128x128-block fp32 scales, bf16 activations.
* ``offload_decode_bf16``  d=4096, E=128, top-8 softmax, F=1536; 32 HBM slots;
                           T=32 tokens per step for 256 steps; router logits
                           biased by a Zipf(1.1) log-prior over a seed-permuted
                           expert order that is re-drawn every 64 steps.
* ``mixtral_prefill_mxfp4`` the Mixtral-shaped prefill layer with MXFP4 expert
                           weights (the experts' fp32 draws converted to MXFP4);
                           activations reach the experts as MXFP8.
* ``offload_decode_mxfp4`` the same layer and stream with MXFP4 expert weights
                           (FP4 E2M1 codes, one E8M0 scale per 32 inputs of an
                           output column), bf16 router and activations.

Draws: ``numpy.random.default_rng([seed, stream, index])``. Stream 0 holds the
weights (one index per tensor, so any expert can be drawn on its own), stream 1
the activation batches, stream 2 the Zipf epochs. Weights are normal with mean
0 and standard deviation 1/sqrt(fan_in) (fan_in = d for the router, the shared
gate and W_gate/W_up, F for W_down); activations are N(0, 1). Values are drawn
in fp32 and then rounded to the storage dtype.
"""
from __future__ import annotations

import math
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, replace

import numpy as np

__all__ = [
    "LayerConfig", "CONFIGS", "get_config", "to_bf16_bits", "quantize_e4m3_blocks", "quantize_mxfp4",
    "gen_router", "gen_shared_gate", "gen_select_bias", "gen_expert", "gen_experts",
    "gen_shared", "gen_x", "zipf_logit_bias",
]

STREAM_W, STREAM_X, STREAM_ZIPF = 0, 1, 2
ID_ROUTER, ID_SHARED_GATE, ID_SELECT_BIAS, ID_SHARED0, ID_EXPERT0 = 0, 1, 2, 3, 16


@dataclass(frozen=True)
class LayerConfig:
    name: str
    T: int
    d: int
    E: int
    k: int
    F: int
    dtype: str                 # "f32" | "bf16" | "fp8" | "mxfp4"
    score_fn: str              # "softmax" | "sigmoid"
    seed: int
    renormalize: int = 1
    route_scale: float = 1.0
    n_groups: int = 1
    topk_groups: int = 1
    group_topn: int = 0
    F_shared: int = 0
    shared_gate: bool = False  # sigmoid scalar gate on the shared expert
    select_bias: bool = False  # per-expert bias added to the selection key
    select_bias_std: float = 0.1
    n_slots: int = 0           # offload: experts held in the HBM slot pool
    steps: int = 0             # offload: decode steps per run
    zipf_alpha: float = 0.0
    zipf_epoch: int = 0

    @property
    def act_dtype(self) -> str:
        return "f32" if self.dtype == "f32" else "bf16"

    def with_T(self, T: int) -> "LayerConfig":
        return replace(self, T=T)


CONFIGS = {
    "tiny_fp32": LayerConfig("tiny_fp32", T=16, d=128, E=8, k=2, F=256, dtype="f32",
                             score_fn="softmax", seed=1),
    "mixtral_prefill_bf16": LayerConfig("mixtral_prefill_bf16", T=4096, d=4096, E=8, k=2,
                                        F=14336, dtype="bf16", score_fn="softmax", seed=2),
    "qwen_decode_bf16": LayerConfig("qwen_decode_bf16", T=8, d=2048, E=60, k=4, F=1408,
                                    dtype="bf16", score_fn="softmax", seed=3, F_shared=5632,
                                    shared_gate=True),
    "dsv3_prefill_fp8": LayerConfig("dsv3_prefill_fp8", T=8192, d=7168, E=256, k=8, F=2048,
                                    dtype="fp8", score_fn="sigmoid", seed=4, route_scale=2.5,
                                    n_groups=8, topk_groups=4, group_topn=2, F_shared=2048,
                                    select_bias=True),
    "offload_decode_bf16": LayerConfig("offload_decode_bf16", T=32, d=4096, E=128, k=8, F=1536,
                                       dtype="bf16", score_fn="softmax", seed=5, n_slots=32,
                                       steps=256, zipf_alpha=1.1, zipf_epoch=64),
    "mixtral_prefill_mxfp4": LayerConfig("mixtral_prefill_mxfp4", T=4096, d=4096, E=8, k=2, F=14336,
                                         dtype="mxfp4", score_fn="softmax", seed=2),
    "offload_decode_mxfp4": LayerConfig("offload_decode_mxfp4", T=32, d=4096, E=128, k=8, F=1536,
                                        dtype="mxfp4", score_fn="softmax", seed=5, n_slots=32,
                                        steps=256, zipf_alpha=1.1, zipf_epoch=64),
}


def get_config(config_name: str, **overrides) -> LayerConfig:
    return replace(CONFIGS[config_name], **overrides)


def stack_configs(cfg: LayerConfig, n_layers: int) -> list:
    """Per-layer configs of a synthetic stack of n_layers copies of cfg: layer l draws its router,
    activations and Zipf epochs from seed cfg.seed + 101*l (the expert weights may be shared)."""
    return [replace(cfg, seed=cfg.seed + 101 * l) for l in range(n_layers)]


def _rng(*key: int) -> np.random.Generator:
    return np.random.default_rng([int(v) for v in key])


def to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """fp32 -> bf16 bit patterns (uint16), round to nearest even; inputs are finite."""
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)
    return ((u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)).astype(np.uint16)


def quantize_e4m3_blocks(w: np.ndarray, block: int = 128):
    """Weight storage for the fp8 workload: per block x block tile, scale = amax/448
    (1 where the tile is all zero) and codes = OCP e4m3fn(w/scale), round to nearest
    even (torch's conversion). Returns (uint8 codes [in,out], fp32 scales [in/b, out/b])."""
    import torch

    n_in, n_out = w.shape
    assert n_in % block == 0 and n_out % block == 0
    wb = w.reshape(n_in // block, block, n_out // block, block)
    amax = np.abs(wb).max(axis=(1, 3)).astype(np.float32)
    scale = np.where(amax > 0, amax / np.float32(448.0), np.float32(1.0)).astype(np.float32)
    scaled = (wb / scale[:, None, :, None]).astype(np.float32).reshape(n_in, n_out)
    codes = torch.from_numpy(np.clip(scaled, -448.0, 448.0)).to(torch.float8_e4m3fn)
    return codes.view(torch.uint8).numpy(), scale


# FP4 E2M1 magnitudes of the codes 0..7 (sign in bit 3)
_FP4_MAG = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0], dtype=np.float64)


def quantize_mxfp4(w: np.ndarray, block: int = 32):
    """Weight storage for the MXFP4 workload (the OCP MX conversion): per output column and
    block of `block` consecutive inputs, shared exponent X = floor(log2(amax)) - 2 (the
    largest E2M1 exponent), clamped to the E8M0 range (X = -127 for an all-zero block);
    codes = E2M1(w / 2^X) rounded to the nearest magnitude, ties to the even code, saturated
    at 6. Returns (uint8 codes [in, out], one code per byte, uint8 E8M0 scales [in/b, out])."""
    n_in, n_out = w.shape
    assert n_in % block == 0
    wb = w.astype(np.float64).reshape(n_in // block, block, n_out)
    amax = np.abs(wb).max(axis=1)
    with np.errstate(divide="ignore"):
        X = np.where(amax > 0, np.floor(np.log2(np.where(amax > 0, amax, 1.0))) - 2, -127)
    X = np.clip(X, -127, 127).astype(np.int64)
    y = np.abs(wb) / np.ldexp(1.0, X)[:, None, :]
    y = np.minimum(y, 6.0)
    hi = np.minimum(np.searchsorted(_FP4_MAG, y, side="left"), 7)
    lo = np.maximum(hi - 1, 0)
    d_lo, d_hi = y - _FP4_MAG[lo], _FP4_MAG[hi] - y
    code = np.where((d_hi < d_lo) | ((d_hi == d_lo) & (hi % 2 == 0)), hi, lo)
    code = np.where(_FP4_MAG[hi] == y, hi, code)
    code = code | (np.signbit(wb).astype(np.int64) << 3)
    return code.reshape(n_in, n_out).astype(np.uint8), (X + 127).astype(np.uint8)


def _store(w32: np.ndarray, dtype: str):
    if dtype == "f32":
        return w32.astype(np.float32)
    if dtype == "bf16":
        return to_bf16_bits(w32)
    if dtype == "fp8":
        return quantize_e4m3_blocks(w32)
    if dtype == "mxfp4":
        return quantize_mxfp4(w32)
    raise ValueError(dtype)


def _normal(shape, std, *key):
    return (_rng(*key).standard_normal(shape, dtype=np.float32) * np.float32(std)).astype(np.float32)


def gen_router(cfg: LayerConfig):
    """W_r [d, E] in the activation dtype (the router runs in bf16 for the fp8 workload)."""
    w = _normal((cfg.d, cfg.E), 1.0 / math.sqrt(cfg.d), cfg.seed, STREAM_W, ID_ROUTER)
    return _store(w, cfg.act_dtype)


def gen_shared_gate(cfg: LayerConfig):
    """w_sg [d] for the shared expert's sigmoid scalar gate (activation dtype)."""
    w = _normal((cfg.d,), 1.0 / math.sqrt(cfg.d), cfg.seed, STREAM_W, ID_SHARED_GATE)
    return _store(w, cfg.act_dtype)


def gen_select_bias(cfg: LayerConfig) -> np.ndarray:
    """Per-expert selection bias [E] fp32, N(0, select_bias_std^2)."""
    return _normal((cfg.E,), cfg.select_bias_std, cfg.seed, STREAM_W, ID_SELECT_BIAS)


def _ffn_weights(cfg: LayerConfig, F: int, base_id: int):
    wg = _normal((cfg.d, F), 1.0 / math.sqrt(cfg.d), cfg.seed, STREAM_W, base_id)
    wu = _normal((cfg.d, F), 1.0 / math.sqrt(cfg.d), cfg.seed, STREAM_W, base_id + 1)
    wd = _normal((F, cfg.d), 1.0 / math.sqrt(F), cfg.seed, STREAM_W, base_id + 2)
    return tuple(_store(w, cfg.dtype) for w in (wg, wu, wd))


def gen_expert(cfg: LayerConfig, e: int):
    """Expert e's (W_gate [d,F], W_up [d,F], W_down [F,d]) in storage format. For fp8 and
    mxfp4 each entry is a (codes, scales) pair."""
    return _ffn_weights(cfg, cfg.F, ID_EXPERT0 + 3 * e)


def gen_experts(cfg: LayerConfig, experts=None, threads: int = 8):
    experts = range(cfg.E) if experts is None else experts
    with ThreadPoolExecutor(max(1, threads)) as ex:
        return list(ex.map(lambda e: gen_expert(cfg, e), experts))


def gen_shared(cfg: LayerConfig):
    """The always-on shared expert's weights (same formats as gen_expert)."""
    assert cfg.F_shared > 0
    return _ffn_weights(cfg, cfg.F_shared, ID_SHARED0)


def gen_x(cfg: LayerConfig, i: int = 0, T: int | None = None):
    """Activation batch i: X [T, d] ~ N(0,1) in the activation dtype."""
    T = cfg.T if T is None else T
    return _store(_normal((T, cfg.d), 1.0, cfg.seed, STREAM_X, i), cfg.act_dtype)


def zipf_logit_bias(cfg: LayerConfig, step: int) -> np.ndarray:
    """Zipf(alpha) log-prior [E] fp32 for decode step `step`. Epoch = step // zipf_epoch; the
    epoch's permutation of expert ids gives each expert a rank r = 1 + its position, and the
    bias is log p(r) = -alpha*ln(r) - ln(H_{E,alpha})."""
    ep = step // cfg.zipf_epoch
    perm = _rng(cfg.seed, STREAM_ZIPF, ep).permutation(cfg.E)
    rank = np.empty(cfg.E, dtype=np.float64)
    rank[perm] = np.arange(1, cfg.E + 1, dtype=np.float64)
    h = np.sum(np.arange(1, cfg.E + 1, dtype=np.float64) ** (-cfg.zipf_alpha))
    return (-cfg.zipf_alpha * np.log(rank) - np.log(h)).astype(np.float32)
