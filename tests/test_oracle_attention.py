"""Pins for the oracle's float64 paged attention (CPU only)."""
import math

import numpy as np
import pytest

from oracle import attention, cache, e4m3
import workloads


def logical_pools(case, mode="per_tensor"):
    pools = cache.new_pools(case.num_pages, case.num_kv_heads, case.head_dim)
    cache.cache_write(pools, case.k, case.v, case.slots, mode)
    return cache.dequantized(pools, "k"), cache.dequantized(pools, "v")


def brute_force_decode(q, k_rows, v_rows, seq_lens, G, window, sm):
    """Pure-Python loops over logical token rows: q [B][Hq][D], k_rows[b][j][g][d]."""
    B, Hq, D = len(q), len(q[0]), len(q[0][0])
    out = [[[0.0] * D for _ in range(Hq)] for _ in range(B)]
    for b in range(B):
        L = seq_lens[b]
        lo = max(0, L - window) if window > 0 else 0
        for h in range(Hq):
            g = h // G
            s = []
            for j in range(lo, L):
                acc = 0.0
                for d in range(D):
                    acc += float(q[b][h][d]) * float(k_rows[b][j][g][d])
                s.append(acc * sm)
            if not s:
                continue
            m = max(s)
            w = [math.exp(x - m) for x in s]
            tot = sum(w)
            for d in range(D):
                out[b][h][d] = sum(w[i] * float(v_rows[b][lo + i][g][d])
                                   for i in range(len(w))) / tot
    return np.array(out)


def per_seq_rows(case, pool):
    rows = []
    for b in range(len(case.seq_lens)):
        rows.append(attention.gather(pool, case.block_table[b], int(case.seq_lens[b])))
    return rows


# ---- pins ---------------------------------------------------------------------

def pin_brute_force(decode_fn, window):
    case = workloads.make_decode_case(11, [19, 33, 1], 6, 2, 16, table="perm",
                                      extra_pages=2)
    kp, vp = logical_pools(case, "per_token_head")
    _, qh = cache.quantize_q(case.q, 1.0)
    got = decode_fn(qh, kp, vp, case.block_table, case.seq_lens, window=window)
    want = brute_force_decode(qh, per_seq_rows(case, kp), per_seq_rows(case, vp),
                              case.seq_lens.tolist(), 3, window, 1 / math.sqrt(16))
    assert np.max(np.abs(got - want)) <= 1e-12


def pin_gqa_grouping(decode_fn):
    """Each KV head's values are constant (= its index), so every output row tells
    which KV head the query head read: h // G."""
    B, Hq, Hkv, D, L = 1, 8, 4, 8, 32
    rng = np.random.default_rng(5)
    P = L // 16
    bt = np.arange(P, dtype=np.int32)[None]
    kp = rng.standard_normal((P, Hkv, 16, D))
    vp = np.zeros((P, Hkv, 16, D))
    for g in range(Hkv):
        vp[:, g] = g
    q = rng.standard_normal((B, Hq, D))
    out = decode_fn(q, kp, vp, bt, np.array([L]), window=0)
    for h in range(Hq):
        assert np.allclose(out[0, h], h // (Hq // Hkv), atol=1e-12)


def pin_equal_keys_mean(decode_fn):
    rng = np.random.default_rng(6)
    P, D, L = 3, 16, 40
    kp = np.tile(rng.standard_normal((1, 1, 1, D)), (P, 1, 16, 1))
    vp = rng.standard_normal((P, 1, 16, D))
    bt = np.array([[2, 0, 1]], np.int32)
    q = rng.standard_normal((1, 2, D))
    out = decode_fn(q, kp, vp, bt, np.array([L]), window=0)
    rows = attention.gather(vp, bt[0], L)[:, 0]
    assert np.allclose(out[0, 0], rows.mean(axis=0), atol=1e-12, rtol=0)
    assert np.allclose(out[0, 1], rows.mean(axis=0), atol=1e-12, rtol=0)


def pin_dominant_key(decode_fn):
    rng = np.random.default_rng(9)
    P, D, L = 4, 32, 60
    kp = rng.standard_normal((P, 1, 16, D)) * 0.1
    vp = rng.standard_normal((P, 1, 16, D))
    bt = np.array([[3, 1, 0, 2]], np.int32)
    q = rng.standard_normal((1, 1, D))
    star = 37
    page, off = bt[0][star // 16], star % 16
    # score gap: q . k* / sqrt(D) = 40 |q|, far above every other key's score
    kp[page, 0, off] = q[0, 0] / np.linalg.norm(q[0, 0]) * 40 * math.sqrt(D)
    out = decode_fn(q, kp, vp, bt, np.array([L]), window=0)
    assert np.allclose(out[0, 0], vp[page, 0, off], atol=1e-9, rtol=0)


def pin_window(decode_fn):
    case = workloads.make_decode_case(12, [50, 7], 2, 1, 8, table="perm")
    kp, vp = logical_pools(case)
    q = case.q.astype(np.float64)
    # W = 1: only the current token
    out = decode_fn(q, kp, vp, case.block_table, case.seq_lens, window=1)
    for b, L in enumerate(case.seq_lens):
        last = attention.gather(vp, case.block_table[b], int(L))[-1, 0]
        assert np.allclose(out[b, :], last, atol=1e-12)
    # W >= seq_len: same as full attention
    full = decode_fn(q, kp, vp, case.block_table, case.seq_lens, window=0)
    big = decode_fn(q, kp, vp, case.block_table, case.seq_lens, window=50)
    assert np.array_equal(full, big)
    # W = 8 equals full attention over the last 8 rows placed in a fresh cache
    w8 = decode_fn(q, kp, vp, case.block_table, case.seq_lens, window=8)
    b = 0
    krow = attention.gather(kp, case.block_table[b], 50)[-8:, 0]
    vrow = attention.gather(vp, case.block_table[b], 50)[-8:, 0]
    ref = attention.attend_rows(q[b], krow, vrow, [0, 0], [7, 7], 1 / math.sqrt(8))
    assert np.allclose(w8[b], ref, atol=1e-12)


def pin_page_permutation(decode_fn):
    case = workloads.make_decode_case(13, [45, 16], 4, 2, 16, table="identity",
                                      extra_pages=2)
    kp, vp = logical_pools(case, "per_token_head")
    q = case.q.astype(np.float64)
    a = decode_fn(q, kp, vp, case.block_table, case.seq_lens, window=0)
    perm = np.random.default_rng(1).permutation(case.num_pages)
    inv = np.argsort(perm)
    kp2, vp2 = kp[perm], vp[perm]               # physical page p moves to inv[p]
    bt2 = inv[case.block_table].astype(np.int32)
    b = decode_fn(q, kp2, vp2, bt2, case.seq_lens, window=0)
    assert np.array_equal(a, b)


# ---- tests --------------------------------------------------------------------

@pytest.mark.parametrize("window", [0, 5])
def test_brute_force(window):
    pin_brute_force(attention.decode, window)


def test_gqa_grouping():
    pin_gqa_grouping(attention.decode)


def test_equal_keys_mean():
    pin_equal_keys_mean(attention.decode)


def test_dominant_key():
    pin_dominant_key(attention.decode)


def test_window():
    pin_window(attention.decode)


def test_page_permutation():
    pin_page_permutation(attention.decode)


@pytest.mark.parametrize("mode", ["per_tensor", "per_token_head"])
def test_tiny_decode_workload_brute_force(mode):
    """The tiny-decode workload (1 x 256 tokens, 4 q / 1 KV head, head_dim 64) in
    both scale modes against pure-Python loops."""
    case = workloads.tiny_decode()
    kp, vp = logical_pools(case, mode)
    _, qh = cache.quantize_q(case.q, 1.0)
    got = attention.decode(qh, kp, vp, case.block_table, case.seq_lens)
    want = brute_force_decode(qh, per_seq_rows(case, kp), per_seq_rows(case, vp),
                              [256], 4, 0, 1 / 8.0)
    assert np.max(np.abs(got - want)) <= 1e-12


def test_zero_length_gives_zeros():
    case = workloads.make_decode_case(14, [0, 20], 2, 1, 8, table="perm", extra_pages=1)
    kp, vp = logical_pools(case)
    out = attention.decode(case.q, kp, vp, case.block_table, case.seq_lens)
    assert not out[0].any() and out[1].any()


def test_lossless_grid_equals_unquantized():
    """K/V/Q on the e4m3 grid with scale 1.0: attention over the dequantised cache
    equals attention over the raw values exactly."""
    case = workloads.make_decode_case(15, [40], 4, 2, 16, table="perm")
    table = e4m3.decode_table()
    grid = table[np.isfinite(table)]
    rng = np.random.default_rng(2)
    grid = grid[np.abs(grid) <= 8]
    case.k = rng.choice(grid, size=case.k.shape).astype(np.float32)
    case.v = rng.choice(grid, size=case.v.shape).astype(np.float32)
    q = rng.choice(grid, size=case.q.shape).astype(np.float32)
    kp, vp = logical_pools(case)
    _, qh = cache.quantize_q(q, 1.0)
    assert np.array_equal(qh, q.astype(np.float64))
    raw_k = np.zeros_like(kp)
    raw_v = np.zeros_like(vp)
    page, off = case.slots // 16, case.slots % 16
    raw_k[page, :, off] = case.k
    raw_v[page, :, off] = case.v
    a = attention.decode(qh, kp, vp, case.block_table, case.seq_lens)
    b = attention.decode(q, raw_k, raw_v, case.block_table, case.seq_lens)
    assert np.array_equal(a, b)


def test_prefill_last_row_equals_decode():
    case = workloads.make_prefill_case(16, [30, 0, 17], [5, 9, 1], 4, 2, 32,
                                       table="perm")
    pools = cache.new_pools(case.num_pages, 2, 32)
    cache.cache_write(pools, case.k, case.v, case.slots, "per_token_head")
    kp, vp = cache.dequantized(pools, "k"), cache.dequantized(pools, "v")
    _, qh = cache.quantize_q(case.q, 1.0)
    out = attention.prefill(qh, case.cu_q_lens, kp, vp, case.block_table,
                            case.seq_lens, causal=True)
    last = case.cu_q_lens[1:] - 1
    dec = attention.decode(qh[last], kp, vp, case.block_table, case.seq_lens)
    assert np.allclose(out[last], dec, atol=1e-13, rtol=0)
    # first new row of the sequence with no context sees exactly one key
    r = case.cu_q_lens[1]
    v0 = attention.gather(vp, case.block_table[1], 1)[0]
    for h in range(4):
        assert np.allclose(out[r, h], v0[h // 2], atol=1e-13)


def test_prefill_brute_force_rows():
    case = workloads.make_prefill_case(17, [21], [6], 4, 1, 8, table="perm",
                                       window=0)
    pools = cache.new_pools(case.num_pages, 1, 8)
    cache.cache_write(pools, case.k, case.v, case.slots, "per_tensor")
    kp, vp = cache.dequantized(pools, "k"), cache.dequantized(pools, "v")
    q = case.q.astype(np.float64)
    for window in (0, 4):
        out = attention.prefill(q, case.cu_q_lens, kp, vp, case.block_table,
                                case.seq_lens, causal=True, window=window)
        krows = attention.gather(kp, case.block_table[0], 27)[:, 0]
        vrows = attention.gather(vp, case.block_table[0], 27)[:, 0]
        for i in range(6):
            pos = 21 + i
            lo = max(0, pos - window + 1) if window else 0
            for h in range(4):
                s = [sum(q[i, h, d] * krows[j, d] for d in range(8)) / math.sqrt(8)
                     for j in range(lo, pos + 1)]
                m = max(s)
                w = [math.exp(x - m) for x in s]
                ref = [sum(w[t] * vrows[lo + t, d] for t in range(len(w))) / sum(w)
                       for d in range(8)]
                assert np.allclose(out[i, h], ref, atol=1e-12, rtol=0)


def test_spread_brute_force_and_special_cases():
    """sum_j w_j |v_j - o| against pure-Python loops; one visible key gives 0; equal
    scores give the plain mean absolute deviation of V about its mean."""
    rng = np.random.default_rng(5)
    q = rng.standard_normal((3, 6))
    k = rng.standard_normal((9, 6))
    v = rng.standard_normal((9, 6))
    lo, hi = [0, 2, 4], [8, 5, 4]
    out, dev = attention.attend_rows(q, k, v, lo, hi, 0.5, spread=True)
    for r in range(3):
        js = range(lo[r], hi[r] + 1)
        s = [0.5 * sum(q[r, d] * k[j, d] for d in range(6)) for j in js]
        m = max(s)
        w = [math.exp(x - m) for x in s]
        tot = sum(w)
        o = [sum(wi * v[j, d] for wi, j in zip(w, js)) / tot for d in range(6)]
        ref = [sum(wi * abs(v[j, d] - o[d]) for wi, j in zip(w, js)) / tot
               for d in range(6)]
        assert np.allclose(out[r], o, atol=1e-13, rtol=0)
        assert np.allclose(dev[r], ref, atol=1e-13, rtol=0)
    assert np.all(dev[2] == 0.0)                     # a single visible key
    _, dev_eq = attention.attend_rows(np.zeros((1, 6)), k, v, [0], [8], 1.0, spread=True)
    assert np.allclose(dev_eq[0], np.mean(np.abs(v - v.mean(axis=0)), axis=0),
                       atol=1e-14, rtol=0)


def test_weight_error_bound_brute_force():
    """attend_rows' bound under per-key weight errors: for tiny rows, every corner of
    the box of relative errors (each weight scaled by 1 - e_j or 1 + e_j, then the
    mean renormalised) moves the output by at most the bound, and the worst corner
    comes within second order of it; zero errors give zero, a constant error r gives
    r / (1 - r) times the spread, and the gap handed to the function is the key's
    log2-domain distance below the row maximum."""
    import itertools
    rng = np.random.default_rng(9)
    for trial in range(6):
        n = 5
        q = rng.standard_normal((1, 4))
        k = rng.standard_normal((n, 4))
        v = rng.standard_normal((n, 4))
        e = rng.uniform(0.0, 0.02, n) if trial % 2 else rng.uniform(0.0, 0.3, n)
        seen = {}

        def fn(gap, js):
            seen["gap"], seen["js"] = np.array(gap), np.array(js)
            return e[np.asarray(js)]
        out, bound = attention.attend_rows(q, k, v, [0], [n - 1], 0.7, weight_error=fn)
        s = 0.7 * (q[0] @ k.T)
        assert np.allclose(seen["gap"], (s - s.max()) / math.log(2.0), atol=1e-12)
        assert list(seen["js"]) == list(range(n))
        w = np.exp(s - s.max())
        worst = np.zeros(4)
        for signs in itertools.product((-1.0, 1.0), repeat=n):
            w2 = w * (1.0 + np.array(signs) * e)
            worst = np.maximum(worst, np.abs(w2 @ v / w2.sum() - out[0]))
        assert np.all(worst <= bound[0] + 1e-15)
        # the numerator's worst case is one corner (signs of v_j - o per channel);
        # only the denominator's 1 - e_j is not attained at the same time
        assert np.all(worst >= bound[0] * (1.0 - e.max()) / (1.0 + e.max()) - 1e-15)
    # special cases
    q = rng.standard_normal((2, 4))
    k = rng.standard_normal((7, 4))
    v = rng.standard_normal((7, 4))
    _, z = attention.attend_rows(q, k, v, [0, 0], [6, 3], 1.0,
                                 weight_error=lambda g, j: np.zeros(len(j)))
    assert np.all(z == 0.0)
    r = 0.05
    _, b = attention.attend_rows(q, k, v, [0, 0], [6, 3], 1.0,
                                 weight_error=lambda g, j: np.full(len(j), r))
    _, sp = attention.attend_rows(q, k, v, [0, 0], [6, 3], 1.0, spread=True)
    assert np.allclose(b, r / (1.0 - r) * sp, rtol=1e-12, atol=0)
    _, inf = attention.attend_rows(q, k, v, [0, 0], [6, 3], 1.0,
                                   weight_error=lambda g, j: np.ones(len(j)))
    assert np.all(np.isinf(inf))


# ---- mutation tests -------------------------------------------------------------

def test_mutants_are_caught():
    # GQA by h % Hkv instead of h // G
    def decode_modulo(q, kp, vp, bt, sl, window=0, sm_scale=None):
        q = np.asarray(q, np.float64)
        B, Hq, D = q.shape
        Hkv = kp.shape[1]
        out = np.zeros_like(q)
        for b in range(B):
            L = int(sl[b])
            k = attention.gather(kp, bt[b], L)
            v = attention.gather(vp, bt[b], L)
            for h in range(Hq):
                out[b, h] = attention.attend_rows(q[b, h][None], k[:, h % Hkv],
                                                  v[:, h % Hkv], [0], [L - 1],
                                                  1 / math.sqrt(D))[0]
        return out
    with pytest.raises(AssertionError):
        pin_gqa_grouping(decode_modulo)

    # softmax scale dropped
    def decode_no_scale(q, kp, vp, bt, sl, window=0, sm_scale=None):
        return attention.decode(q, kp, vp, bt, sl, window=window, sm_scale=1.0)
    with pytest.raises(AssertionError):
        pin_brute_force(decode_no_scale, 0)

    # page index taken from the logical page number (block table ignored)
    def decode_no_table(q, kp, vp, bt, sl, window=0, sm_scale=None):
        ident = np.arange(bt.size, dtype=np.int32).reshape(bt.shape)
        return attention.decode(q, kp, vp, ident, sl, window=window)
    with pytest.raises(AssertionError):
        pin_brute_force(decode_no_table, 0)

    # window off by one (W+1 keys)
    def decode_window_plus_one(q, kp, vp, bt, sl, window=0, sm_scale=None):
        return attention.decode(q, kp, vp, bt, sl, window=window + 1 if window else 0)
    with pytest.raises(AssertionError):
        pin_window(decode_window_plus_one)
