"""CPU oracle for the 8-bit floating-point (OCP E4M3FN) quantiser used by the
fp8 mode of the linear layers.

TEST INFRASTRUCTURE ONLY (see oracle/block.py).

The pages name fp8 training of the linear layers (flicky.cc course page
"nanochat: свой ChatGPT от токенизатора до чата", repository map row for
nanochat/fp8.py; leaderboard row "d26 slightly undertrained +fp8" in the
README mirror) but not its format or recipe.  Reading taken: OCP E4M3FN
(1 sign, 4 exponent bits with bias 7, 3 mantissa bits; exponent field 15
with mantissa 7 is NaN, no infinities; largest finite 448), current
per-tensor scaling s = amax / 448 (s = 1 when amax = 0), round to nearest
with ties to an even code, saturating at +-448.

Quantisation decisions are taken in float32, as the kernels take them:
inv = fp32(448) / fp32(amax); scaled = fp32(fp32(x) * inv); code =
nearest-even E4M3 of scaled.  In the block, the quantiser's input is the
tensor as the bf16 pipeline holds it: round_bf16 gives that rounding
(float32, then nearest-even to 8 significant bits).
"""
from __future__ import annotations

import numpy as np

E4M3_MAX = 448.0


def e4m3_decode(code: int) -> float:
    """Value of one 8-bit code, from the format's definition."""
    code = int(code) & 0xFF
    sign = -1.0 if code & 0x80 else 1.0
    e = (code >> 3) & 0xF
    m = code & 0x7
    if e == 0xF and m == 0x7:
        return float("nan")
    if e == 0:
        return sign * (m / 8.0) * 2.0 ** (1 - 7)
    return sign * (1.0 + m / 8.0) * 2.0 ** (e - 7)


def e4m3_table() -> np.ndarray:
    """Values of all 256 codes, indexed by code."""
    return np.array([e4m3_decode(c) for c in range(256)])


_POS = e4m3_table()[:0x7F]   # codes 0..126: the finite non-negative values, increasing


def e4m3_encode(x: np.ndarray) -> np.ndarray:
    """Nearest E4M3 code to each value, ties to the even code, saturating to
    the largest finite magnitude.  Input float64 (exact comparisons)."""
    x = np.asarray(x, dtype=np.float64)
    mag = np.minimum(np.abs(x), E4M3_MAX)
    hi = np.searchsorted(_POS, mag, side="left")          # first value >= mag
    hi = np.clip(hi, 0, len(_POS) - 1)
    lo = np.clip(hi - 1, 0, len(_POS) - 1)
    d_lo = mag - _POS[lo]
    d_hi = _POS[hi] - mag
    pick_hi = (d_hi < d_lo) | ((d_hi == d_lo) & (hi % 2 == 0))
    code = np.where(pick_hi, hi, lo).astype(np.int64)
    code = np.where(mag == _POS[hi], hi, code)
    # the sign is kept, as in IEEE conversions: negative values that round
    # to zero give the negative-zero code 0x80
    return (code | np.where(np.signbit(x), 0x80, 0)).astype(np.uint8)


def round_bf16(x: np.ndarray) -> np.ndarray:
    """Nearest bfloat16 (1 sign, 8 exponent, 7 stored mantissa bits) of each
    value, ties to even, via float32; returned as float64."""
    b = np.ascontiguousarray(np.asarray(x, dtype=np.float32)).view(np.uint32).astype(np.uint64)
    b = (b + 0x7FFF + ((b >> 16) & 1)) & 0xFFFF0000
    return b.astype(np.uint32).view(np.float32).astype(np.float64)


def e4m3_values(codes: np.ndarray) -> np.ndarray:
    return e4m3_table()[np.asarray(codes, dtype=np.int64)]


def quantize_tensor(x: np.ndarray, amax=None):
    """Per-tensor current scaling: returns (codes uint8, scale float32) with
    x ~= value(codes) * scale.  Decisions in float32 as stated above.

    amax: the tensor's absolute maximum when x is only part of the tensor
    the scale belongs to (default: max |x|).  amax = 0 gives inv = s = 1, and
    the values (all zeros, of either sign) go through the same rounding, so
    -0 keeps its sign code 0x80."""
    x32 = np.asarray(x, dtype=np.float32)
    if amax is None:
        amax = np.max(np.abs(x32)) if x32.size else 0.0
    amax = np.float32(amax)
    if amax > 0:
        inv = np.float32(E4M3_MAX) / amax
        scale = np.float32(amax / np.float32(E4M3_MAX))
    else:
        inv = scale = np.float32(1.0)
    scaled = (x32 * inv).astype(np.float32)
    return e4m3_encode(scaled.astype(np.float64)), scale


def fake_quant(x: np.ndarray, amax=None) -> np.ndarray:
    """Round trip through the quantiser, as float64."""
    codes, s = quantize_tensor(x, amax)
    return e4m3_values(codes) * np.float64(s)
