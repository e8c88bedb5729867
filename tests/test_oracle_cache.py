"""Pins for the oracle's quantising cache write, Q quantisation and scale rules."""
import os

import numpy as np
import pytest

from oracle import cache, e4m3, scales
import workloads

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "scale_resolution.txt")


# ---- per-token-head scale -----------------------------------------------------

def pin_scale_closed_form(scale_fn):
    rng = np.random.default_rng(7)
    x = workloads.bf16_round(rng.standard_normal((200, 64)).astype(np.float32) * 3)
    s = scale_fn(x)
    amax = np.abs(x).max(axis=1)
    # closed form in float32: IEEE division of two float32 values
    for i in range(len(s)):
        assert s[i] == np.float32(np.float32(amax[i]) / np.float32(448.0))
    # a row whose amax is exactly 448 * 2^k gets scale 2^k
    row = np.zeros((1, 64), np.float32)
    row[0, 5] = -448.0 * 0.25
    assert scale_fn(row)[0] == np.float32(0.25)


def pin_scale_invariants(quantize_rows):
    rng = np.random.default_rng(8)
    x = workloads.bf16_round(rng.standard_normal((500, 128)).astype(np.float32))
    x[3] = 0.0                           # a zero row
    codes, s = quantize_rows(x, "per_token_head")
    assert s[3] == 1.0 and not codes[3].any()
    nz = np.abs(x).max(axis=1) > 0
    mag = codes & 0x7F
    # every non-zero row holds a +-448 code at its amax, and no NaN code
    assert np.all((mag[nz] == 0x7E).any(axis=1))
    assert not np.any(mag == 0x7F)
    # the code at the amax position has the row's sign there
    i = np.abs(x).argmax(axis=1)
    r = np.arange(len(x))
    assert np.all((codes[r, i] == 0xFE) == (x[r, i] < 0))


def test_scale_closed_form():
    pin_scale_closed_form(cache.per_token_head_scale)


def test_scale_invariants():
    pin_scale_invariants(cache.quantize_rows)


def test_scale_nan_row_propagates():
    x = np.ones((2, 8), np.float32)
    x[1, 3] = np.nan
    s = cache.per_token_head_scale(x)
    assert s[0] == np.float32(1.0) / np.float32(448.0)
    assert np.isnan(s[1])
    codes, _ = cache.quantize_rows(x, "per_token_head")
    assert np.all((codes[1] & 0x7F) == 0x7F)


def test_lossless_on_grid_scale_one():
    """Values already on the e4m3 grid at scale 1.0 come back unchanged."""
    table = e4m3.decode_table()
    grid = table[~np.isnan(table)].astype(np.float32)
    codes, s = cache.quantize_rows(grid[None, :], "per_tensor", 1.0)
    assert np.array_equal(cache.dequantize(codes, s[:, None])[0], grid.astype(np.float64))


def test_quantize_double_rounding_is_float32_quotient():
    """x / s is rounded to float32 first: where the exact quotient lies just off a
    midpoint between two codes but its float32 rounding lands on the midpoint, the
    code is the even neighbour (a single exact rounding would pick the other side
    about half the time)."""
    from fractions import Fraction
    table = e4m3.decode_table()
    found = 0
    for c in range(0x08, 0x7D):
        mid = (table[c] + table[c + 1]) / 2
        even = c if c % 2 == 0 else c + 1
        for s in (np.float32(1.99), np.float32(3.97), np.float32(0.2497),
                  np.float32(0.0123)):
            x0 = np.float32(mid * float(s))
            for x in (np.nextafter(x0, np.float32(-np.inf), dtype=np.float32), x0,
                      np.nextafter(x0, np.float32(np.inf), dtype=np.float32)):
                exact = Fraction(float(x)) / Fraction(float(s))
                if float(np.float32(x / s)) == mid and exact != Fraction(mid):
                    found += 1
                    assert cache.quantize(np.array([x]), s)[0] == even
    assert found > 20


def test_quantize_nan_quotient_sign_of_input():
    x = np.array([np.inf, -np.inf, 1.0], np.float32)
    got = cache.quantize(x, np.float32(np.inf))
    assert got.tolist() == [0x7F, 0xFF, 0x00]


# ---- paged cache write ----------------------------------------------------------

def test_cache_write_scatter_and_skip():
    case = workloads.make_decode_case(3, [37, 5, 0, 16], 4, 2, 64, table="perm",
                                      extra_pages=3)
    pools = cache.new_pools(case.num_pages, 2, 64)
    slots = case.slots.copy()
    slots[4] = -1                                      # skipped token
    cache.cache_write(pools, case.k, case.v, slots, "per_token_head")
    for t in range(len(slots)):
        page, off = divmod(int(case.slots[t]), 16)
        if t == 4:
            assert np.isnan(pools["k_scales"][page, :, off]).all()
            continue
        codes, s = cache.quantize_rows(case.k[t], "per_token_head")
        assert np.array_equal(pools["k_codes"][page, :, off], codes)
        assert np.array_equal(pools["k_scales"][page, :, off], s)
        codes, s = cache.quantize_rows(case.v[t], "per_token_head")
        assert np.array_equal(pools["v_codes"][page, :, off], codes)


def test_per_kv_head_lossless_on_scaled_grid():
    """Per-KV-head scale arrays ("vLLM FP8 KV-Cache and Attention Quantization
    Update", section "Kernel and fusion optimizations"): rows of head h that are
    e4m3 grid values times s_h (powers of two, so the products are exact) come back
    unchanged, each head at its own scale, and the codes equal the grid's codes."""
    table = e4m3.decode_table()
    grid = table[~np.isnan(table)].astype(np.float32)[::3]        # 84 values
    s = np.array([0.25, 2.0, 0.0078125], np.float32)
    x = grid[None, None, :] * s[None, :, None]                     # [1][3][84]
    codes, scales = cache.quantize_rows(x, "per_kv_head", s)
    assert np.array_equal(scales[0], s)
    assert np.array_equal(codes[0], np.broadcast_to(e4m3.encode(grid), (3, grid.size)))
    assert np.array_equal(cache.dequantize(codes, scales[..., None]), x.astype(np.float64))


def test_per_kv_head_is_per_tensor_per_head():
    """Head h of a per-KV-head write equals a per-tensor write of that head alone at
    s_h; with every s_h equal the whole write equals the per-tensor one."""
    case = workloads.make_decode_case(9, [40, 3], 8, 4, 64, table="perm")
    s = np.array([0.5, 0.03, 1.0, 0.125], np.float32)
    pools = cache.new_pools(case.num_pages, 4, 64)
    cache.cache_write(pools, case.k, case.v, case.slots, "per_kv_head", s, s * 2)
    page, off = case.slots // 16, case.slots % 16
    for h in range(4):
        codes, _ = cache.quantize_rows(case.k[:, h], "per_tensor", float(s[h]))
        assert np.array_equal(pools["k_codes"][page, h, off], codes)
        codes, _ = cache.quantize_rows(case.v[:, h], "per_tensor", float(2 * s[h]))
        assert np.array_equal(pools["v_codes"][page, h, off], codes)
        assert np.all(pools["k_scales"][page, h, off] == s[h])
    same = cache.new_pools(case.num_pages, 4, 64)
    cache.cache_write(same, case.k, case.v, case.slots, "per_kv_head",
                      np.full(4, 0.2, np.float32), np.full(4, 0.3, np.float32))
    ref = cache.new_pools(case.num_pages, 4, 64)
    cache.cache_write(ref, case.k, case.v, case.slots, "per_tensor", 0.2, 0.3)
    for name in ("k_codes", "v_codes"):
        assert np.array_equal(same[name], ref[name])


def test_quantize_q():
    q = np.array([[0.3, -2.0, 500.0]], np.float32)
    codes, qh = cache.quantize_q(q, 0.5)
    assert codes.tolist() == [e4m3.encode(np.float32([0.6, -4.0, 448.0])).tolist()]
    assert np.array_equal(qh, e4m3.decode(codes) * 0.5)


# ---- scale resolution (golden cases from the pages' rules) ------------------------

def read_scale_cases():
    for line in open(GOLDEN):
        line = line.split("#")[0].strip()
        if not line:
            continue
        lhs, rhs = line.split("->")
        mode, *raw = lhs.split()
        yield mode, [float(t) for t in raw], rhs.split()


def test_scale_resolution_golden():
    n = 0
    for mode, raw, rhs in read_scale_cases():
        n += 1
        if rhs == ["error"]:
            with pytest.raises(scales.ScaleError):
                scales.resolve(mode, *raw)
            continue
        s, warn = scales.resolve(mode, *raw)
        want = [float(t) for t in rhs]
        assert [s.q_scale, s.k_scale, s.v_scale, s.prob_scale] == want[:4], raw
        assert warn == int(want[4]), raw
    assert n >= 10


def test_skip_policy():
    assert scales.layer_kv_dtype(128, scales.SKIP_SLIDING_WINDOW) == "bf16"
    assert scales.layer_kv_dtype(0, scales.SKIP_SLIDING_WINDOW) == "fp8"
    assert scales.layer_kv_dtype(128, 0) == "fp8"
    assert scales.layer_kv_dtype(0, 0) == "fp8"


# ---- mutation tests -------------------------------------------------------------

def test_mutants_are_caught():
    # reciprocal multiply instead of division
    def scale_recip(x):
        amax = np.abs(np.asarray(x, np.float32)).max(axis=-1)
        return np.where(amax == 0, 1, amax * np.float32(1.0 / 448.0)).astype(np.float32)
    with pytest.raises(AssertionError):
        pin_scale_closed_form(scale_recip)

    # scale from amax / 240 (the wrong format's max)
    def rows_wrong_max(x, mode, ts=1.0):
        x = np.asarray(x, np.float32)
        amax = np.abs(x).max(axis=-1)
        s = np.where(amax == 0, 1, amax / np.float32(240)).astype(np.float32)
        return cache.quantize(x, s[..., None]), s
    with pytest.raises(AssertionError):
        pin_scale_invariants(rows_wrong_max)
