"""Pins for the oracle's e4m3 table and encoder (CPU only).

Each pin is written as a function of the callable under test so that the mutation
tests at the bottom can show it catches plausible mistakes.
"""
import os

import numpy as np
import pytest
import torch

from oracle import e4m3

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "e4m3_named_values.txt")


def read_named_values():
    rows = []
    for line in open(GOLDEN):
        line = line.split("#")[0].strip()
        if not line:
            continue
        code, val, _src = line.split()
        rows.append((int(code, 16), float(val)))
    return rows


# ---- pins ---------------------------------------------------------------------

def pin_table_named_values(table):
    for code, val in read_named_values():
        if np.isnan(val):
            assert np.isnan(table[code]), hex(code)
        else:
            assert table[code] == val, hex(code)
            assert np.signbit(table[code]) == np.signbit(val), hex(code)


def pin_table_matches_torch(table):
    ref = torch.arange(256, dtype=torch.int32).to(torch.uint8).view(
        torch.float8_e4m3fn).double().numpy()
    assert np.array_equal(np.isnan(table), np.isnan(ref))
    fin = ~np.isnan(ref)
    assert np.array_equal(table[fin], ref[fin])
    assert np.array_equal(np.signbit(table[fin]), np.signbit(ref[fin]))


def pin_sign_magnitude_order(table):
    # inside one sign, code order is value order, one ulp is one code step
    pos = table[0x00:0x7F]
    neg = table[0x80:0xFF]
    assert np.all(np.diff(pos) > 0)
    assert np.all(np.diff(neg) < 0)
    assert np.array_equal(-pos, neg)
    # subnormal grid step 2^-9 (codes 0x00..0x08 evenly spaced)
    assert np.all(np.diff(table[0:9]) == 2.0 ** -9)


def pin_round_trip(encode, table):
    finite = np.array([c for c in range(256) if not np.isnan(table[c])], np.uint8)
    assert len(finite) == 254
    assert np.array_equal(encode(table[finite].astype(np.float32)), finite)
    nan_codes = encode(np.array([np.nan, -np.nan], np.float32))
    assert np.isnan(table[nan_codes]).all()


def pin_midpoints(encode, table):
    """Every midpoint between neighbouring non-negative codes goes to the even code;
    one float32 ulp either side goes to the nearer code."""
    for c in range(0, 0x7E):
        a, b = table[c], table[c + 1]
        mid = np.float32((a + b) / 2)
        assert float(mid) == (a + b) / 2           # midpoints are exact in float32
        even = c if c % 2 == 0 else c + 1
        got = encode(np.array([mid, -mid], np.float32))
        assert got[0] == even, (hex(c), float(mid))
        assert got[1] == (even | 0x80) or (even == 0 and got[1] == 0x80)
        lo = np.nextafter(mid, np.float32(-np.inf), dtype=np.float32)
        hi = np.nextafter(mid, np.float32(np.inf), dtype=np.float32)
        assert encode(np.array([lo], np.float32))[0] == c
        assert encode(np.array([hi], np.float32))[0] == c + 1


def pin_saturation(encode):
    x = np.array([448.0, 449.0, 464.0, 480.0, 1e30, np.inf, -448.0, -1e9, -np.inf],
                 np.float32)
    assert encode(x).tolist() == [0x7E] * 6 + [0xFE] * 3


def all_bf16_values():
    bits = np.arange(65536, dtype=np.uint32) << 16
    return bits.view(np.float32)


def torch_saturating_cast(x_f32):
    t = torch.from_numpy(np.ascontiguousarray(x_f32, np.float32))
    return t.clamp(-448.0, 448.0).to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def pin_exhaustive_bf16(encode, scale):
    """All 65,536 bf16 patterns divided by ``scale`` in float32, against torch's
    saturating cast of the same float32 quotients."""
    x = all_bf16_values()
    with np.errstate(all="ignore"):
        qt = (x / np.float32(scale)).astype(np.float32)
    got = encode(qt)
    ref = torch_saturating_cast(qt)
    nan = np.isnan(qt)
    assert np.array_equal(got[~nan], ref[~nan])
    assert np.all((got[nan] & 0x7F) == 0x7F)


# ---- tests --------------------------------------------------------------------

def test_table_named_values():
    pin_table_named_values(e4m3.decode_table())


def test_table_matches_torch():
    pin_table_matches_torch(e4m3.decode_table())


def test_sign_magnitude_order():
    pin_sign_magnitude_order(e4m3.decode_table())


def test_round_trip():
    pin_round_trip(e4m3.encode, e4m3.decode_table())


def test_midpoints():
    pin_midpoints(e4m3.encode, e4m3.decode_table())


def test_saturation():
    pin_saturation(e4m3.encode)


@pytest.mark.parametrize("scale", [1.0, 0.5, 0.0123, 3.0 / 448.0, 1e-3, 7.5])
def test_exhaustive_bf16(scale):
    pin_exhaustive_bf16(e4m3.encode, scale)


def test_negative_zero_and_tiny():
    got = e4m3.encode(np.array([-0.0, -1e-30, 0.0, 2.0 ** -10, -(2.0 ** -10)],
                               np.float32))
    assert got.tolist() == [0x80, 0x80, 0x00, 0x00, 0x80]


# ---- mutation tests: each pin must reject a plausible mistake -------------------

def _encode_round_half_up(x):
    # mistake: ties away from zero instead of ties to even
    x = np.asarray(x, np.float64)
    a = np.abs(x)
    out = e4m3.encode(x)
    table = e4m3.decode_table()
    for i, ai in np.ndenumerate(a):
        if np.isfinite(ai) and ai < 448:
            c = out[i] & 0x7F
            if c < 0x7E and ai == (table[c] + table[c + 1]) / 2:
                out[i] = (out[i] & 0x80) | (c + 1)
    return out


def _encode_truncate(x):
    # mistake: truncation toward zero
    table = e4m3.decode_table()
    x = np.asarray(x, np.float64)
    pos = table[:0x7F]
    idx = np.searchsorted(pos, np.minimum(np.abs(x), 448.0), side="right") - 1
    return (idx.astype(np.int64) | np.where(np.signbit(x), 0x80, 0)).astype(np.uint8)


def _table_wrong_bias():
    codes = np.arange(256)
    e = (codes >> 3) & 0xF
    m = codes & 7
    v = np.where(e == 0, m * 2.0 ** -9, (1 + m / 8) * 2.0 ** (e - 8))
    return np.where(codes & 0x80, -v, v)


def test_mutants_are_caught():
    table = e4m3.decode_table()
    with pytest.raises(AssertionError):
        pin_midpoints(_encode_round_half_up, table)
    with pytest.raises(AssertionError):
        pin_exhaustive_bf16(_encode_truncate, 1.0)
    with pytest.raises(AssertionError):
        pin_table_named_values(_table_wrong_bias())
    with pytest.raises(AssertionError):
        pin_table_matches_torch(_table_wrong_bias())
