"""Number formats of the stored tensors, written from the format definitions.

TEST INFRASTRUCTURE ONLY: this package is the CPU oracle. Only ``tests/``,
``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of ``bench.py`` may
import it; the product library never does.

Formats
-------
* binary32 / binary64: numpy's IEEE types (library primitives).
* bfloat16: the upper 16 bits of an IEEE binary32 (1 sign, 8 exponent bits with
  bias 127, 7 stored mantissa bits).  Rounding from any real value is
  round-to-nearest-even at 8 significant bits.
* fp8 e4m3fn (the OCP "E4M3" format): 1 sign, 4 exponent bits with bias 7,
  3 mantissa bits; exponent field 0 is subnormal (value m * 2^-9); there is no
  infinity, and the single NaN pattern per sign is exponent 15 with mantissa 7,
  so the largest finite magnitude is 1.75 * 2^8 = 448.

The low-precision key cache these formats serve is motivated by the V4 report
digest (https://gitcode.csdn.net/69eb1ea054b52172bc6fc291.html, section 七:
the indexer's QK path is run in low precision because its cached activations are
loaded at every long-context step) and by the FP8/FP4 KV-cache remark in the
structured summary (https://www.10100.com/article/149217299, section 五).
"""
from __future__ import annotations

import numpy as np

E4M3_MAX = 448.0


def round_rne(v, precision_bits: int, min_exp: int) -> np.ndarray:
    """Round real values (given as float64) to a binary format, nearest-even.

    ``precision_bits`` counts the implicit leading bit; ``min_exp`` is the
    exponent of the smallest normal number.  Values below it land on the
    subnormal grid 2^(min_exp - precision_bits + 1).  No overflow handling:
    callers clamp or flag values beyond their format's largest finite number.
    Every step is exact in float64 (scaling by powers of two and ``rint``).
    """
    v = np.asarray(v, dtype=np.float64)
    a = np.abs(v)
    _, ex = np.frexp(a)  # a = f * 2**ex with f in [0.5, 1)
    e = np.maximum(ex - 1, min_exp)  # exponent of the leading bit
    ulp = np.ldexp(np.ones_like(a), e - (precision_bits - 1))
    r = np.rint(a / ulp) * ulp  # numpy rint rounds halves to even
    return np.copysign(r, v)


# ----------------------------------------------------------------------------- bf16

BF16_MAX = float(np.ldexp(2.0 - 2.0 ** -7, 127))


def bf16_bits_to_f64(bits) -> np.ndarray:
    """Decode raw bf16 bit patterns (uint16) to float64 (exact)."""
    u = np.asarray(bits).astype(np.uint32) << np.uint32(16)
    with np.errstate(invalid="ignore"):  # NaN patterns stay NaN; only the warning is silenced
        return u.view(np.float32).astype(np.float64)


def round_to_bf16(v) -> np.ndarray:
    """Round real values once to the nearest bf16 value (returned as float64)."""
    r = round_rne(v, 8, -126)
    r = np.where(np.abs(r) > BF16_MAX, np.copysign(np.inf, r), r)
    return np.where(np.isnan(np.asarray(v, np.float64)), np.nan, r)


def f64_to_bf16_bits(v) -> np.ndarray:
    """bf16 bit patterns of ``round_to_bf16(v)`` (the rounded value is exact in binary32)."""
    r = round_to_bf16(v).astype(np.float32)
    return (r.view(np.uint32) >> np.uint32(16)).astype(np.uint16)


def round_to_f32(v) -> np.ndarray:
    """Round float64 values once to binary32 (IEEE conversion), returned as float64."""
    return np.asarray(v, dtype=np.float64).astype(np.float32).astype(np.float64)


# ----------------------------------------------------------------------------- e4m3


def _e4m3_table() -> np.ndarray:
    """Value of every e4m3fn code 0..255, from the field definitions."""
    vals = np.empty(256, dtype=np.float64)
    for code in range(256):
        s = (code >> 7) & 1
        e = (code >> 3) & 0xF
        m = code & 0x7
        if e == 0xF and m == 0x7:
            val = np.nan
        elif e == 0:
            val = m * 2.0 ** -9
        else:
            val = (1.0 + m / 8.0) * 2.0 ** (e - 7)
        vals[code] = -val if s else val
    return vals


E4M3_VALUES = _e4m3_table()
# Codes 0..126 are the finite non-negative values, and they increase with the
# code (exponent field above mantissa field), so a rounded magnitude finds its
# code by binary search.
_E4M3_POS_VALUES = E4M3_VALUES[:0x7F]
assert np.all(np.diff(_E4M3_POS_VALUES) > 0)


def e4m3_decode(codes) -> np.ndarray:
    """Decode e4m3fn codes (uint8) to float64 values (exact)."""
    return E4M3_VALUES[np.asarray(codes, dtype=np.uint8)]


def e4m3_encode(v) -> np.ndarray:
    """Encode real values to e4m3fn codes, round-to-nearest-even.

    Magnitudes in (448, 464] round to 448 (464 is the midpoint to the next,
    unrepresentable, step and ties go to the even mantissa 448); larger
    magnitudes and NaN give the NaN code.  Negative zero keeps its sign bit.
    """
    v = np.asarray(v, dtype=np.float64)
    a = np.abs(round_rne(v, 4, -6))
    finite = ~np.isnan(v) & (a <= E4M3_MAX)
    a_ok = np.where(finite, a, 0.0)
    code = np.searchsorted(_E4M3_POS_VALUES, a_ok).astype(np.int64)
    assert np.all(_E4M3_POS_VALUES[code] == a_ok), "rounded value not on the e4m3 grid"
    code = np.where(finite, code, 0x7F)
    code = np.where(np.signbit(v), code | 0x80, code)
    return code.astype(np.uint8)


def e4m3_quantize_rows(r32: np.ndarray):
    """Per-row absmax quantisation of binary32 rows to e4m3fn with a binary32 scale.

    The decisions are taken in binary32 arithmetic, as the quantiser on the GPU
    takes them: ``scale = f32(max_i |r_i| / 448)``, the maximum taken over the
    elements that are not NaN, and ``scale = 1`` where that quotient is 0 (an
    all-zero row, or one whose largest magnitude is below 448 * 2^-150, where
    the quotient underflows); then ``code_i = e4m3_rne(f32(r_i / scale))``.  A
    NaN element gets a NaN code; an infinite element makes the scale infinite,
    so every stored value of its row is NaN (0 * inf or inf / inf).  Returns
    ``(codes uint8 [N, d], scale float32 [N], stored float64 [N, d])`` where
    ``stored = decode(code) * scale`` is exact in float64.
    """
    r32 = np.asarray(r32, dtype=np.float32)
    amax = np.max(np.where(np.isnan(r32), np.float32(0.0), np.abs(r32)), axis=-1)
    with np.errstate(under="ignore"):
        scale = (amax / np.float32(E4M3_MAX)).astype(np.float32)  # binary32 division
    scale = np.where(scale == 0, np.float32(1.0), scale).astype(np.float32)
    with np.errstate(invalid="ignore"):
        y = (r32 / scale[..., None]).astype(np.float32)  # binary32 division
    codes = e4m3_encode(y.astype(np.float64))
    with np.errstate(invalid="ignore"):
        stored = e4m3_decode(codes) * scale.astype(np.float64)[..., None]
    return codes, scale, stored
