"""Pins for the oracle's float64 paged query-key logits (CPU only)."""
import numpy as np
import pytest

from oracle import cache, logits
import workloads


def pools_of(case, mode="per_token_head"):
    pools = cache.new_pools(case.num_pages, case.num_kv_heads, case.head_dim)
    cache.cache_write(pools, case.k, case.v, case.slots, mode)
    return cache.dequantized(pools, "k")


def small_case(seed=3, seq_lens=(1, 16, 17, 40), rows=(1, 2, 3, 4), hq=4, hkv=2, d=8,
               causal_rows=True):
    return workloads.make_logits_case(seed, list(seq_lens), list(rows), hq, hkv, d,
                                      table="perm", causal_rows=causal_rows, extra_pages=3)


def pin_brute_force(fn):
    """Pure-Python dot products over the logical token rows, each row found from its
    slot (page, offset) rather than through the block table."""
    case = small_case()
    kp = pools_of(case)
    out_len = int(case.seq_lens.max()) + 2
    got = fn(case.q, case.cu_rows, case.row_lens, kp, case.block_table, out_len)
    G = case.q.shape[1] // case.num_kv_heads
    starts = np.concatenate([[0], np.cumsum(case.seq_lens)[:-1]])
    for b in range(len(case.seq_lens)):
        for r in range(case.cu_rows[b], case.cu_rows[b + 1]):
            for h in range(case.q.shape[1]):
                for j in range(out_len):
                    if j >= case.row_lens[r]:
                        assert got[r, h, j] == -np.inf
                        continue
                    slot = int(case.slots[starts[b] + j])
                    krow = kp[slot // 16, h // G, slot % 16]
                    want = 0.0
                    for d in range(case.head_dim):
                        want += float(case.q[r, h, d]) * float(krow[d])
                    assert abs(got[r, h, j] - want) <= 1e-12 * (1 + abs(want))


def pin_one_hot(fn):
    """q = e_d picks channel d of the key: a lookup, no arithmetic."""
    case = small_case(seed=5)
    kp = pools_of(case)
    q = np.zeros_like(case.q)
    R, Hq, D = q.shape
    for r in range(R):
        for h in range(Hq):
            q[r, h, (3 * r + h) % D] = 1.0
    out_len = int(case.seq_lens.max())
    got = fn(q, case.cu_rows, case.row_lens, kp, case.block_table, out_len)
    G = Hq // case.num_kv_heads
    for b in range(len(case.seq_lens)):
        for r in range(case.cu_rows[b], case.cu_rows[b + 1]):
            for h in range(Hq):
                j = np.arange(case.row_lens[r])
                pages = case.block_table[b][j // 16]
                want = kp[pages, h // G, j % 16, (3 * r + h) % D]
                assert np.array_equal(got[r, h, :len(j)], want)


def pin_gqa_constant_heads(fn):
    """Key head g filled with g + 1: logits = (g + 1) * sum(q), g = h // (Hq / Hkv)."""
    case = small_case(seed=7, hq=8, hkv=4)
    kp = np.zeros((case.num_pages, 4, 16, case.head_dim))
    for g in range(4):
        kp[:, g] = g + 1.0
    out_len = int(case.seq_lens.max())
    got = fn(case.q, case.cu_rows, case.row_lens, kp, case.block_table, out_len)
    for r in range(case.q.shape[0]):
        for h in range(8):
            n = case.row_lens[r]
            want = (h // 2 + 1) * float(np.sum(case.q[r, h].astype(np.float64)))
            assert np.allclose(got[r, h, :n], want, rtol=1e-12, atol=1e-12)


def pin_visibility():
    """Finite entries per (row, head) = row_lens[r]; an empty row is all -inf."""
    case = small_case(seed=9, seq_lens=(0, 5, 33), rows=(2, 1, 3), causal_rows=True)
    kp = pools_of(case)
    got = logits.paged_logits(case.q, case.cu_rows, case.row_lens, kp, case.block_table, 40)
    for r in range(case.q.shape[0]):
        for h in range(case.q.shape[1]):
            assert np.isfinite(got[r, h]).sum() == case.row_lens[r]
            assert np.all(np.isfinite(got[r, h, :case.row_lens[r]]))
    assert list(case.row_lens) == [0, 0, 5, 31, 32, 33]


def pin_page_permutation(fn):
    """Moving physical pages and rewriting the table to match changes nothing."""
    case = small_case(seed=11)
    kp = pools_of(case)
    out_len = int(case.seq_lens.max())
    base = fn(case.q, case.cu_rows, case.row_lens, kp, case.block_table, out_len)
    perm = np.random.default_rng(1).permutation(case.num_pages)
    kp2 = np.empty_like(kp)
    kp2[perm] = kp
    bt2 = perm[case.block_table]
    moved = fn(case.q, case.cu_rows, case.row_lens, kp2, bt2, out_len)
    assert np.array_equal(base, moved)


def pin_bilinear(fn):
    """logits(a q1 + q2) = a logits(q1) + logits(q2) on the visible entries."""
    case = small_case(seed=13)
    kp = pools_of(case)
    rng = np.random.default_rng(2)
    q1 = rng.standard_normal(case.q.shape)
    q2 = rng.standard_normal(case.q.shape)
    out_len = int(case.seq_lens.max())
    args = (case.cu_rows, case.row_lens, kp, case.block_table, out_len)
    lhs = fn(2.5 * q1 + q2, *args)
    rhs = 2.5 * fn(q1, *args) + fn(q2, *args)
    fin = np.isfinite(lhs)
    assert np.array_equal(fin, np.isfinite(rhs))
    assert np.allclose(lhs[fin], rhs[fin], rtol=1e-12, atol=1e-12)


def test_brute_force():
    pin_brute_force(logits.paged_logits)


def test_one_hot():
    pin_one_hot(logits.paged_logits)


def test_gqa_constant_heads():
    pin_gqa_constant_heads(logits.paged_logits)


def test_visibility():
    pin_visibility()


def test_narrow_output_is_a_prefix():
    """An output narrower than the visible keys holds the first out_len of them."""
    case = small_case(seed=15)
    kp = pools_of(case)
    wide = logits.paged_logits(case.q, case.cu_rows, case.row_lens, kp, case.block_table, 48)
    narrow = logits.paged_logits(case.q, case.cu_rows, case.row_lens, kp, case.block_table, 20)
    assert np.array_equal(narrow, wide[:, :, :20])


def test_page_permutation():
    pin_page_permutation(logits.paged_logits)


def test_bilinear():
    pin_bilinear(logits.paged_logits)


# ---- mutation tests -------------------------------------------------------------

def test_mutants_are_caught():
    # key head by h % Hkv instead of h // G
    def modulo_heads(q, cu, rl, kp, bt, out_len):
        Hkv = kp.shape[1]
        q = np.asarray(q, np.float64)
        out = np.full((q.shape[0], q.shape[1], out_len), -np.inf)
        for b in range(len(cu) - 1):
            for r in range(cu[b], cu[b + 1]):
                n = int(rl[r])
                k = logits.gather(kp, bt[b], n)
                for h in range(q.shape[1]):
                    out[r, h, :n] = k[:, h % Hkv] @ q[r, h]
        return out
    with pytest.raises(AssertionError):
        pin_gqa_constant_heads(modulo_heads)

    # block table ignored (logical page number used as the physical one)
    def no_table(q, cu, rl, kp, bt, out_len):
        ident = np.arange(bt.size).reshape(bt.shape)
        return logits.paged_logits(q, cu, rl, kp, ident, out_len)
    with pytest.raises(AssertionError):
        pin_brute_force(no_table)

    # one key too many visible
    def plus_one(q, cu, rl, kp, bt, out_len):
        return logits.paged_logits(q, cu, np.asarray(rl) + 1, kp, bt, out_len)
    with pytest.raises(AssertionError):
        pin_brute_force(plus_one)

    # every row of a request given the first row's length
    def first_row_len(q, cu, rl, kp, bt, out_len):
        rl = np.asarray(rl).copy()
        for b in range(len(cu) - 1):
            rl[cu[b]:cu[b + 1]] = rl[cu[b]] if cu[b + 1] > cu[b] else 0
        return logits.paged_logits(q, cu, rl, kp, bt, out_len)
    with pytest.raises(AssertionError):
        pin_brute_force(first_row_len)

    # token offset inside the page reversed
    def reversed_offset(q, cu, rl, kp, bt, out_len):
        return logits.paged_logits(q, cu, rl, kp[:, :, ::-1, :], bt, out_len)
    with pytest.raises(AssertionError):
        pin_one_hot(reversed_offset)

    # channels of the key read in the wrong order
    def flipped_channels(q, cu, rl, kp, bt, out_len):
        return logits.paged_logits(q, cu, rl, kp[..., ::-1], bt, out_len)
    with pytest.raises(AssertionError):
        pin_one_hot(flipped_channels)
