"""Number formats used by the layer's inputs (oracle side, test infrastructure only).

bf16: the upper 16 bits of an IEEE binary32 value; decoding is exact.

OCP E4M3 (the "fn" variant of the OCP 8-bit floating point specification,
as used for fp8 MoE weights): 1 sign bit, 4 exponent bits with bias 7, 3
mantissa bits. Exponent field 0 encodes subnormals (m/8 * 2^-6); the pattern
S.1111.111 is NaN; there are no infinities; the largest finite magnitude is
1.75 * 2^8 = 448. Encoding here is round-to-nearest-even with saturation to
+-448, the conversion the fp8 workload uses for activations.

OCP MXFP4 (the OCP Microscaling Formats specification, as used for 4-bit MoE
expert weights): elements are FP4 E2M1, 1 sign bit, 2 exponent bits with bias 1
and 1 mantissa bit, exponent field 0 being subnormal (m/2), so the magnitudes are
0, 0.5, 1, 1.5, 2, 3, 4 and 6; every 32 consecutive elements along the reduction
axis share one E8M0 scale, the power of two 2^(e-127) (e = 255 is NaN).

The pages list FP8 among the weight formats an MoE offload engine must carry
("guqiong96/Lvllm", section "Highlights") and require the quantisation scales
to travel with the weights as one unit ("Running 35B MoE Models on 8GB GPUs",
section "Technical Insight"); the exact format is the reading above. They also
name 4-bit weights (MXFP4 and NVFP4, "guqiong96/Lvllm", section "Highlights"), of
which MXFP4 is the one taken here.

OCP MXFP8 (same specification): E4M3 elements sharing one E8M0 scale per 32
consecutive values. It is the activation format taken where MXFP4 experts run on
the block-scaled matrix instructions, which multiply two MX operands; the
conversion follows the specification: the shared exponent is floor(log2 of the
block's largest magnitude) minus 8 (the exponent of E4M3's largest normal), and
each element is the nearest E4M3 value of v / 2^X, saturated at +-448.
"""
from __future__ import annotations

import numpy as np

E4M3_MAX = 448.0


def decode_bf16(bits: np.ndarray) -> np.ndarray:
    """bf16 bit patterns (uint16) -> float64, exact."""
    u = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    with np.errstate(invalid="ignore"):
        return u.view(np.float32).astype(np.float64)


def _e4m3_magnitude(code: int) -> float:
    """Value of the 7-bit magnitude field (sign stripped) per the OCP E4M3 definition."""
    exp = (code >> 3) & 0xF
    man = code & 0x7
    if exp == 15 and man == 7:
        return float("nan")
    if exp == 0:
        return (man / 8.0) * 2.0 ** (1 - 7)
    return (1.0 + man / 8.0) * 2.0 ** (exp - 7)


# Magnitudes of codes 0x00..0x7E (0x7F is NaN); strictly increasing in the code.
_E4M3_POS = np.array([_e4m3_magnitude(c) for c in range(0x7F)], dtype=np.float64)


def e4m3_table() -> np.ndarray:
    """float64 value of each of the 256 codes (NaN for 0x7F and 0xFF)."""
    t = np.empty(256, dtype=np.float64)
    for c in range(256):
        m = _e4m3_magnitude(c & 0x7F)
        t[c] = -m if (c & 0x80) else m
    return t


_E4M3_TABLE = e4m3_table()


def decode_e4m3(codes: np.ndarray) -> np.ndarray:
    """uint8 codes -> float64."""
    return _E4M3_TABLE[np.asarray(codes, dtype=np.uint8)]


def encode_e4m3(x: np.ndarray) -> np.ndarray:
    """Finite values -> uint8 codes: clamp to +-448, then the nearest representable
    magnitude; an exact halfway case goes to the code with an even mantissa (its
    lowest bit clear). The sign bit follows the input's sign (so -0.0 and small
    negatives that round to zero give 0x80)."""
    x = np.asarray(x, dtype=np.float64)
    if np.isnan(x).any():
        raise ValueError("encode_e4m3: NaN input")
    mag = np.minimum(np.abs(x), E4M3_MAX)
    hi = np.searchsorted(_E4M3_POS, mag, side="left")          # first code with value >= mag
    hi = np.minimum(hi, len(_E4M3_POS) - 1)
    lo = np.maximum(hi - 1, 0)
    d_lo = mag - _E4M3_POS[lo]
    d_hi = _E4M3_POS[hi] - mag
    pick_hi = (d_hi < d_lo) | ((d_hi == d_lo) & (hi % 2 == 0))
    code = np.where(pick_hi, hi, lo)
    code = np.where(_E4M3_POS[hi] == mag, hi, code)            # exact hit
    sign = np.signbit(x).astype(np.uint8) << np.uint8(7)
    return (code.astype(np.uint8) | sign).astype(np.uint8)


def quantize_rows_e4m3(x: np.ndarray, block: int = 128):
    """Per-token, per-`block`-column activation quantisation, all in IEEE fp32:
    a = max|x| over the block, scale = a / 448 (1 when a == 0),
    q = e4m3(clamp(x / scale, +-448)). Returns (uint8 codes [R, C], fp32 scales [R, C/block]).

    The fp32 steps fix the quantised codes bit for bit, so a device implementation that
    divides in IEEE fp32 and rounds to nearest even must produce the same codes."""
    x32 = np.asarray(x, dtype=np.float32)
    R, C = x32.shape
    if C % block:
        raise ValueError("quantize_rows_e4m3: columns must be a multiple of the block")
    xb = x32.reshape(R, C // block, block)
    amax = np.abs(xb).max(axis=2)
    scale = np.where(amax > 0, amax / np.float32(E4M3_MAX), np.float32(1.0)).astype(np.float32)
    y = (xb / scale[:, :, None]).astype(np.float32)
    y = np.clip(y, -E4M3_MAX, E4M3_MAX)
    return encode_e4m3(y.reshape(R, C)), scale


def dequantize_rows(codes: np.ndarray, scales: np.ndarray, block: int = 128) -> np.ndarray:
    """Inverse of quantize_rows_e4m3 in float64: value = e4m3(code) * scale of its block."""
    v = decode_e4m3(codes)
    R, C = v.shape
    return (v.reshape(R, C // block, block) * scales.astype(np.float64)[:, :, None]).reshape(R, C)


def dequantize_weight_blocks(codes: np.ndarray, scales: np.ndarray, block: int = 128) -> np.ndarray:
    """Weights stored as e4m3 codes [in, out] with one fp32 scale per block x block tile
    [in/block, out/block] -> float64 [in, out]."""
    v = decode_e4m3(codes)
    n_in, n_out = v.shape
    s = scales.astype(np.float64)
    return (v.reshape(n_in // block, block, n_out // block, block) * s[:, None, :, None]).reshape(n_in, n_out)


# ------------------------------------------------------------------ MXFP4 --
MX_BLOCK = 32


def _e2m1_magnitude(code: int) -> float:
    """Value of the 3-bit magnitude field (sign stripped) per the E2M1 definition."""
    e = (code >> 1) & 3
    m = code & 1
    if e == 0:
        return 0.5 * m                       # subnormal: m/2 * 2^(1 - bias)
    return (1.0 + 0.5 * m) * 2.0 ** (e - 1)  # normal: (1 + m/2) * 2^(e - bias)


def e2m1_table() -> np.ndarray:
    """float64 value of each of the 16 FP4 E2M1 codes (code 8 is -0.0)."""
    return np.array([(-1.0 if c & 8 else 1.0) * _e2m1_magnitude(c & 7) for c in range(16)], dtype=np.float64)


_E2M1_TABLE = e2m1_table()


def decode_e2m1(codes: np.ndarray) -> np.ndarray:
    """FP4 codes (one per uint8, values 0..15) -> float64."""
    c = np.asarray(codes, dtype=np.uint8)
    if (c > 15).any():
        raise ValueError("decode_e2m1: codes are 4-bit")
    return _E2M1_TABLE[c]


def decode_e8m0(e: np.ndarray) -> np.ndarray:
    """E8M0 scale bytes -> float64 2^(e - 127); 255 is NaN."""
    e = np.asarray(e, dtype=np.uint8).astype(np.int64)
    v = np.ldexp(1.0, e - 127)
    return np.where(e == 255, np.nan, v)


def dequantize_mxfp4_weight(codes: np.ndarray, scales: np.ndarray) -> np.ndarray:
    """Weights stored as FP4 codes [in, out] (one code per byte) with one E8M0 scale per
    32 consecutive inputs of an output column, scales [in/32, out] -> float64 [in, out]."""
    v = decode_e2m1(codes)
    n_in, n_out = v.shape
    if n_in % MX_BLOCK:
        raise ValueError("dequantize_mxfp4_weight: the input dimension must be a multiple of 32")
    s = decode_e8m0(scales)
    return (v.reshape(n_in // MX_BLOCK, MX_BLOCK, n_out) * s[:, None, :]).reshape(n_in, n_out)


# ------------------------------------------------------------------ MXFP8 --
E4M3_EMAX = 8   # exponent of E4M3's largest normal: 448 = 1.75 * 2^8


def mx_shared_exponent(amax: np.ndarray, emax: int) -> np.ndarray:
    """Shared exponent X of MX blocks with largest magnitudes `amax`: floor(log2(amax)) - emax,
    clamped to the E8M0 range [-127, 127]; -127 for an all-zero block. floor(log2) is read off
    frexp, which is exact (amax = m 2^e with m in [0.5, 1) gives e - 1)."""
    a = np.asarray(amax, dtype=np.float64)
    _, e = np.frexp(np.where(a > 0, a, 1.0))
    X = np.where(a > 0, e.astype(np.int64) - 1 - emax, -127)
    return np.clip(X, -127, 127)


def quantize_rows_mxfp8(x: np.ndarray, block: int = MX_BLOCK):
    """Rows -> MXFP8: per `block` consecutive values of a row the shared exponent X
    (mx_shared_exponent with E4M3's emax 8) and the elements e4m3(v / 2^X), nearest even,
    saturated at +-448 (v / 2^X is exact). Returns (uint8 codes [R, C], uint8 E8M0 exponents
    X + 127 [R, C/block])."""
    v = np.asarray(x, dtype=np.float64)
    R, C = v.shape
    if C % block:
        raise ValueError("quantize_rows_mxfp8: columns must be a multiple of the block")
    vb = v.reshape(R, C // block, block)
    X = mx_shared_exponent(np.abs(vb).max(axis=2), E4M3_EMAX)
    codes = encode_e4m3(np.ldexp(vb, -X[:, :, None]).reshape(R, C))
    return codes, (X + 127).astype(np.uint8)


def dequantize_rows_mxfp8(codes: np.ndarray, exps: np.ndarray, block: int = MX_BLOCK) -> np.ndarray:
    """Inverse of quantize_rows_mxfp8 in float64: e4m3(code) * 2^(exp - 127)."""
    v = decode_e4m3(codes)
    R, C = v.shape
    return (v.reshape(R, C // block, block) * decode_e8m0(exps)[:, :, None]).reshape(R, C)
