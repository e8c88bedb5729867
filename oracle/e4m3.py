"""OCP FP8 E4M3 ("e4m3fn") code table and encoder, written from the format's definition.

Test infrastructure only: see the package docstring for who may import it.

Sources.
  * The cache element type is ``torch.float8_e4m3fn`` ("vLLM Qwen3.8-Flash-Next: FP8
    support for the QSA indexer cache", section "Code analysis", the
    ``indexer_dtype`` parametrisation and the one-ulp comparator).  That comparator's
    comment fixes two properties used as pins: the format is sign-magnitude (inside
    one sign, code order is value order and one ulp is one code step) and the
    subnormal grid step is 2^-9.
  * The quantisation rule x = clamp(round_rne(v / scale), +-448): round to nearest,
    ties to even, saturating at the largest finite magnitude 448.

Bit layout of one code byte: S EEEE MMM, exponent bias 7.
  E = 0        -> (-1)^S * M * 2^-9           (zero and subnormals)
  E = 1..15    -> (-1)^S * (1 + M/8) * 2^(E-7)
  E = 15, M = 7 -> NaN (0x7F and 0xFF); the format has no infinity.

The encoder below works in float64 on values that are exactly float32, using
``frexp`` and ``rint`` (half-to-even).  It shares nothing with the device encoder,
which works on float32 bit patterns.
"""
from __future__ import annotations

import numpy as np

E4M3_MAX = 448.0          # largest finite magnitude, code 0x7E
E4M3_MIN_NORMAL = 2.0 ** -6   # code 0x08
E4M3_MIN_SUBNORMAL = 2.0 ** -9  # code 0x01, also the subnormal grid step
CODE_MAX = 0x7E
CODE_NAN = 0x7F


def decode_table() -> np.ndarray:
    """float64[256]: the value of every code byte (NaN for 0x7F and 0xFF)."""
    codes = np.arange(256, dtype=np.int64)
    sign = np.where(codes & 0x80, -1.0, 1.0)
    e = (codes >> 3) & 0xF
    m = (codes & 0x7).astype(np.float64)
    sub = m * E4M3_MIN_SUBNORMAL
    norm = (1.0 + m / 8.0) * np.exp2((e - 7).astype(np.float64))
    val = sign * np.where(e == 0, sub, norm)
    val[(e == 15) & (codes & 0x7 == 7)] = np.nan
    return val


_TABLE = decode_table()


def decode(codes) -> np.ndarray:
    """Values (float64) of an array of code bytes."""
    return _TABLE[np.asarray(codes, dtype=np.uint8)]


def encode(x) -> np.ndarray:
    """Round-to-nearest-even, saturating encoder: float (exactly float32) -> code byte.

    NaN -> 0x7F with the input's sign bit; |x| >= 448 (and +-inf) -> 0x7E with the
    sign bit; the sign of zero is kept (tiny negatives give 0x80).
    """
    x = np.asarray(x, dtype=np.float64)
    neg = np.signbit(x)
    a = np.abs(x)
    with np.errstate(invalid="ignore", over="ignore"):
        # Subnormal range (a < 2^-6): the grid is n * 2^-9, n = 0..8; n = 8 is the
        # smallest normal code 0x08, so the integer n is the code itself.
        n_sub = np.rint(a * 512.0)
        # Normal range: a = f * 2^k with f in [0.5, 1) -> a = (2f) * 2^(k-1),
        # 2f in [1, 2), three fraction bits kept by rounding (2f - 1) * 8.
        f, k = np.frexp(a)
        e = k.astype(np.int64) - 1
        m = np.rint((2.0 * f - 1.0) * 8.0).astype(np.int64)
        carry = m == 8
        e = e + carry
        m = np.where(carry, 0, m)
        code_norm = ((e + 7) << 3) | m
        code = np.where(a < E4M3_MIN_NORMAL, n_sub.astype(np.int64), code_norm)
        code = np.where(a >= E4M3_MAX, CODE_MAX, code)
        code = np.where(np.isnan(a), CODE_NAN, code)
    code = code.astype(np.int64) | np.where(neg, 0x80, 0)
    return code.astype(np.uint8)
