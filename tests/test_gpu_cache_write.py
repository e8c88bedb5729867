"""GPU parity: e4m3 quantiser and quantising cache write, bit-exact to the oracle."""
import numpy as np
import pytest

import workloads
from oracle import cache as ocache

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module")
def kvq():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import fp8_quantized_paged_amd as k
    return k


from gpu_common import dev, dev_bf16, log, oracle_pools, read_pools, write_cache  # noqa: E402


def all_bf16():
    return (np.arange(65536, dtype=np.uint32) << 16).view(np.float32)


@pytest.mark.parametrize("scale", [1.0, 0.5, 0.0123, 3.0 / 448.0, 7.5, 1e-3, 448.0])
def test_quantize_exhaustive_bf16(kvq, scale):
    x = all_bf16()
    log(f"quantize exhaustive scale={scale}")
    got = kvq.quantize_fp8(dev_bf16(x), scale).cpu().numpy()
    want = ocache.quantize(x, np.float32(scale))
    bad = np.nonzero(got != want)[0]
    assert bad.size == 0, [(hex(int(i) << 16), hex(got[i]), hex(want[i])) for i in bad[:8]]


def test_quantize_ragged_tail(kvq):
    rng = np.random.default_rng(3)
    for n in (1, 7, 9, 1000, 4097):
        x = workloads.bf16_round(rng.standard_normal(n).astype(np.float32) * 30)
        got = kvq.quantize_fp8(dev_bf16(x), 0.25).cpu().numpy()
        assert np.array_equal(got, ocache.quantize(x, np.float32(0.25))), n


def _check_pools(got, want, rows_slots):
    page, off = rows_slots // 16, rows_slots % 16
    for name in ("k_codes", "v_codes"):
        g, w = got[name][page, :, off], want[name][page, :, off]
        assert np.array_equal(g, w), (name, int((g != w).sum()))
    if "k_scales" in got:
        for name in ("k_scales", "v_scales"):
            g, w = got[name][page, :, off], want[name][page, :, off]
            assert np.array_equal(g.view(np.uint32), w.view(np.uint32)), name


@pytest.mark.parametrize("mode", ["per_tensor", "per_token_head"])
def test_cache_write_tiny_decode(kvq, mode):
    case = workloads.tiny_decode()
    log(f"cache_write tiny {mode}")
    c = write_cache(kvq, case, "fp8", mode)
    _check_pools(read_pools(c), oracle_pools(case, mode), case.slots)


@pytest.mark.parametrize("D", [64, 128, 256])
def test_cache_write_ragged_perm(kvq, D):
    case = workloads.make_decode_case(21 + D, [1, 17, 0, 40, 16], 8, 4, D, table="perm",
                                      outliers=4, extra_pages=5)
    for mode, ks, vs in (("per_token_head", 1.0, 1.0), ("per_tensor", 0.37, 2.5)):
        log(f"cache_write ragged D={D} {mode}")
        c = write_cache(kvq, case, "fp8", mode, ks, vs)
        _check_pools(read_pools(c), oracle_pools(case, mode, ks, vs), case.slots)


def test_cache_write_skips_negative_slots_and_strided_rows(kvq):
    case = workloads.make_decode_case(31, [33], 4, 2, 128, table="perm", extra_pages=2)
    c = kvq.PagedCache(case.num_pages, 2, 128, "fp8", "per_token_head")
    slots = case.slots.copy()
    slots[::3] = -1
    # rows embedded in a wider [T][3*H*D] buffer (as K/V come out of a fused QKV)
    T = len(slots)
    wide_k = np.zeros((T, 3, 2, 128), np.float32)
    wide_v = np.zeros_like(wide_k)
    wide_k[:, 1] = case.k
    wide_v[:, 2] = case.v
    kt = dev_bf16(wide_k)
    vt = dev_bf16(wide_v)
    kvq.cache_write(c, kt[:, 1], vt[:, 2], dev(slots), token_stride=3 * 2 * 128)
    got = read_pools(c)
    keep = slots >= 0
    want = ocache.new_pools(case.num_pages, 2, 128)
    ocache.cache_write(want, case.k, case.v, slots, "per_token_head")
    _check_pools(got, want, slots[keep])
    skipped = case.slots[~keep]
    page, off = skipped // 16, skipped % 16
    assert not got["k_codes"][page, :, off].any()
    assert not got["k_scales"][page, :, off].any()


def test_cache_write_edge_values(kvq):
    """Zero rows, NaN/inf entries, tiny values, values above 448 and exact-grid rows."""
    D, H = 64, 2
    rows = np.zeros((8, H, D), np.float32)
    rows[1, 0, 3] = np.nan
    rows[2, 1, :] = np.inf
    rows[2, 1, 5] = -np.inf
    rows[3] = 1e-30
    rows[4] = workloads.bf16_round(np.linspace(-1000, 1000, D, dtype=np.float32))
    rows[5, :, ::2] = -0.0
    rows[6] = workloads.bf16_round(np.float32(2.0) ** np.arange(-20, 44, dtype=np.float32))
    rows[7] = 448.0
    rows = workloads.bf16_round(rows)
    slots = np.arange(8, dtype=np.int64) * 3
    case = workloads.DecodeCase("edge", np.zeros((1, H, D), np.float32), rows, rows[::-1].copy(),
                                np.zeros(8, np.int64), np.arange(8), slots,
                                np.arange(2, dtype=np.int32)[None], np.array([8], np.int32),
                                2, H, D)
    for mode, ks in (("per_token_head", 1.0), ("per_tensor", 1.0), ("per_tensor", 0.001)):
        log(f"cache_write edges {mode} {ks}")
        c = write_cache(kvq, case, "fp8", mode, ks, ks)
        got = read_pools(c)
        want = oracle_pools(case, mode, ks, ks)
        page, off = slots // 16, slots % 16
        for name in ("k_codes", "v_codes"):
            assert np.array_equal(got[name][page, :, off], want[name][page, :, off]), name
        if mode == "per_token_head":
            for name in ("k_scales", "v_scales"):
                g, w = got[name][page, :, off], want[name][page, :, off]
                both_nan = np.isnan(g) & np.isnan(w)
                assert np.array_equal(g[~both_nan].view(np.uint32),
                                      w[~both_nan].view(np.uint32)), name
                assert np.array_equal(np.isnan(g), np.isnan(w)), name


def test_cache_write_bf16_copy(kvq):
    case = workloads.make_decode_case(41, [20, 3], 8, 2, 64, table="perm")
    c = write_cache(kvq, case, "bf16")
    got = read_pools(c)
    page, off = case.slots // 16, case.slots % 16
    assert np.array_equal(got["k"][page, :, off], case.k)
    assert np.array_equal(got["v"][page, :, off], case.v)


def test_cache_write_llama8b_sampled(kvq):
    """Full Llama-3.1-8B-shaped cache (8 x 20,000 tokens, outlier channels), written
    in the bulk configuration; codes and scales compared on sampled tokens."""
    case = workloads.llama8b_decode()
    log("cache_write llama8b full")
    c = write_cache(kvq, case, "fp8", "per_token_head", chunk=1 << 24)
    torch.cuda.synchronize()
    rng = np.random.default_rng(0)
    rows = np.sort(rng.choice(len(case.k), size=4000, replace=False))
    want = oracle_pools(case, "per_token_head", rows=rows)
    _check_pools(read_pools(c), want, case.slots[rows])


@pytest.mark.parametrize("which", ["long_context", "gptoss_full", "gptoss_window",
                                   "hd256_prefill"])
def test_cache_write_full_size_sampled(kvq, which):
    """Codes and scales bit-exact on the other full-size workloads, written in the bulk
    configuration: the 131,072-token cache (per-tensor scale 1.0, the planted key's row
    included), a gpt-oss-shaped full-attention layer (fp8, per-tensor) and window layer
    (bf16 copy), and the head_dim-256 prefill cache (per-token-head) with every one of
    its 8,192 new tokens."""
    rng = np.random.default_rng(11)
    if which == "long_context":
        case, dtype, mode = workloads.long_context_decode(), "fp8", "per_tensor"
        extra = [case.meta["planted_pos"]]
    elif which.startswith("gptoss"):
        case = workloads.gptoss_hybrid_layer(0 if which == "gptoss_full" else 1)
        dtype = kvq.layer_kv_dtype(case.window, kvq.SKIP_SLIDING_WINDOW)
        mode, extra = "per_tensor", []
    else:
        case, dtype, mode = workloads.hd256_prefill(), "fp8", "per_token_head"
        extra = list(case.new_token_rows())
    log(f"cache_write {which} full ({dtype}, {mode})")
    c = write_cache(kvq, case, dtype, mode, chunk=1 << 24)
    torch.cuda.synchronize()
    rows = np.unique(np.concatenate([rng.choice(len(case.k), size=4000, replace=False),
                                     np.asarray(extra, np.int64)]))
    got = read_pools(c)
    if dtype == "bf16":
        page, off = case.slots[rows] // 16, case.slots[rows] % 16
        assert np.array_equal(got["k"][page, :, off], case.k[rows])
        assert np.array_equal(got["v"][page, :, off], case.v[rows])
        return
    want = oracle_pools(case, mode, rows=rows)
    _check_pools(got, want, case.slots[rows])


def _rows_for_maxima(maxima, D):
    """Per-token-head rows: each row's maximum magnitude is one of ``maxima`` (its first
    value, signs alternating between rows), the other D - 1 values run through every
    finite bf16 x with |x| <= that maximum, so every (x, row maximum) pair of the list
    occurs.  Returns float32 [rows][D]."""
    allx = all_bf16()
    rows = []
    for k, a in enumerate(maxima):
        xs = allx[np.isfinite(allx) & (np.abs(allx) <= a)]
        for i in range(0, len(xs), D - 1):
            r = np.zeros(D, np.float32)
            chunk = xs[i:i + D - 1]
            r[1:1 + len(chunk)] = chunk
            r[0] = a if (len(rows) + k) % 2 == 0 else -a
            rows.append(r)
    return np.stack(rows)


@pytest.mark.parametrize("ordered", [True, False])
def test_cache_write_per_token_head_row_maxima(kvq, ordered):
    """Per-token-head codes are bit-exact over every bf16 value against a set of row
    maxima: the ends of the fast-quotient range (2^-100 and the bf16 values beside it,
    the largest finite bf16), a subnormal maximum (division path), 1 and 448, and 40
    seeded maxima across the exponent range.  ordered: slots in page order (the
    whole-page LDS path); otherwise scattered slots (the single-row path)."""
    D, H = 128, 8
    rng = np.random.default_rng(77)
    bits = [0x0D80, 0x0D7F, 0x0D81, 0x0001, 0x3F80, 0x43E0, 0x7F7F]
    bits += list(rng.integers(0x0080, 0x7F7F, size=40))
    maxima = (np.array(bits, dtype=np.uint32) << 16).view(np.float32)
    rows = _rows_for_maxima(maxima, D)
    T = (len(rows) + H - 1) // H
    pad = np.zeros((T * H - len(rows), D), np.float32)
    x = np.concatenate([rows, pad]).reshape(T, H, D)
    v = x[::-1].copy()                       # V: the same rows, other tokens
    P = (T + 15) // 16
    slots = np.arange(T, dtype=np.int64)
    if not ordered:
        slots = rng.permutation(P * 16)[:T].astype(np.int64)
    log(f"per-token-head row maxima: {len(rows)} rows, ordered={ordered}")
    c = kvq.PagedCache(P, H, D, "fp8", "per_token_head")
    kvq.cache_write(c, dev_bf16(x), dev_bf16(v), dev(slots))
    pools = ocache.new_pools(P, H, D)
    ocache.cache_write(pools, x, v, slots, "per_token_head", 1.0, 1.0)
    _check_pools(read_pools(c), pools, slots)


def _mixed_block_slots():
    """Slots for 10 blocks of 16 tokens plus a 7-token tail, each block a different case
    of the whole-page test the write takes per block: whole pages in order (the LDS
    path), in order but one slot off the page boundary, one swapped pair, a skipped
    token (-1) inside a page, a page in reverse, scattered slots; the partial tail is in
    order but shorter than a page (the single-row path)."""
    rng = np.random.default_rng(2024)
    pages = iter(rng.permutation(64)[:40].tolist())  # distinct pages, no slot written twice
    blocks = []
    p = next(pages); blocks.append(16 * p + np.arange(16))                      # run
    p = next(pages); next(pages); blocks.append(16 * p + 1 + np.arange(16))    # off by one
    b = 16 * next(pages) + np.arange(16); b[[5, 6]] = b[[6, 5]]; blocks.append(b)  # swap
    b = 16 * next(pages) + np.arange(16); b[7] = -1; blocks.append(b)          # skip inside
    p = next(pages); blocks.append(16 * p + np.arange(16))                      # run
    blocks.append(16 * next(pages) + np.arange(15, -1, -1))                     # reversed
    p = next(pages); blocks.append(16 * p + np.arange(16))                      # run
    scat = np.array([16 * next(pages) + int(o) for o in rng.integers(0, 16, 16)])
    blocks.append(scat)                                                         # scattered
    blocks.append(16 * next(pages) + np.arange(16))                             # run
    blocks.append(16 * next(pages) + np.arange(16))                             # run
    blocks.append(16 * next(pages) + np.arange(7))                              # tail
    return np.concatenate(blocks).astype(np.int64)


@pytest.mark.parametrize("mode", ["per_token_head", "per_tensor", "bf16"])
def test_cache_write_mixed_page_blocks(kvq, mode):
    """One call whose 16-token blocks alternate between whole pages in order and the
    near misses of that test; every written row bit-exact to the oracle, no other slot
    touched."""
    H, D, P = 2, 128, 64
    slots = _mixed_block_slots()
    T = len(slots)
    rng = np.random.default_rng(5)
    k = workloads.bf16_round(rng.standard_normal((T, H, D)).astype(np.float32) * 3)
    v = workloads.bf16_round(rng.standard_normal((T, H, D)).astype(np.float32) * 3)
    log(f"cache_write mixed page blocks {mode}: {T} tokens")
    dtype = "bf16" if mode == "bf16" else "fp8"
    c = kvq.PagedCache(P, H, D, dtype, "per_tensor" if mode == "bf16" else mode)
    c.k_pages.view(torch.uint8).fill_(0x5A)   # a marker in every byte: untouched slots keep it
    c.v_pages.view(torch.uint8).fill_(0x5A)
    kvq.cache_write(c, dev_bf16(k), dev_bf16(v), dev(slots), 0.5, 0.25)
    got = read_pools(c)
    keep = slots >= 0
    page, off = slots[keep] // 16, slots[keep] % 16
    if mode == "bf16":
        assert np.array_equal(got["k"][page, :, off], k[keep])
        assert np.array_equal(got["v"][page, :, off], v[keep])
    else:
        want = ocache.new_pools(P, H, D)
        ocache.cache_write(want, k, v, slots, mode, 0.5, 0.25)
        _check_pools(got, want, slots[keep])
    # every slot no token was written to still holds the marker
    written = np.zeros(P * 16, bool)
    written[slots[keep]] = True
    untouched = np.nonzero(~written)[0]
    eb = 2 if mode == "bf16" else 1
    kraw = c.k_pages.view(torch.uint8).cpu().numpy().reshape(P, H, 16, D * eb)
    vraw = c.v_pages.view(torch.uint8).cpu().numpy().reshape(P, H, D, 16, eb)
    assert (kraw[untouched // 16, :, untouched % 16] == 0x5A).all()
    assert (vraw[untouched // 16, :, :, untouched % 16] == 0x5A).all()


def _mid_page_slots(seed, starts_lens, pages_per_seq):
    """Slots of several sequences' new tokens, each chunk starting at its own position
    (mostly mid-page) in a permuted page table; the pages of different sequences are
    distinct, so no slot is written twice."""
    rng = np.random.default_rng(seed)
    perm = rng.permutation(len(starts_lens) * pages_per_seq)
    out = []
    for i, (start, n) in enumerate(starts_lens):
        pos = start + np.arange(n)
        pages = perm[i * pages_per_seq:(i + 1) * pages_per_seq]
        out.append(pages[pos // 16] * 16 + pos % 16)
    return np.concatenate(out).astype(np.int64), len(starts_lens) * pages_per_seq


@pytest.mark.parametrize("mode", ["per_token_head", "per_tensor", "bf16"])
@pytest.mark.parametrize("D", [64, 256])
def test_cache_write_mid_page_chunks(kvq, mode, D):
    """Chunks that start mid-page: a 16-token block then ends one page in order and starts
    another (any page of the table) in order -- the two-run store path -- and chunks whose
    blocks straddle sequences (the single-row path).  Bit-exact to the oracle; every slot no
    token was written to keeps its marker (the rows of a page's other tokens survive)."""
    H = 2
    starts_lens = [(1, 16 * 5 + 3), (2, 40), (7, 16 * 3), (8, 37), (13, 70), (15, 16 * 4 + 1),
                   (0, 33)]
    slots, P = _mid_page_slots(77 + D, starts_lens, 8)
    T = len(slots)
    rng = np.random.default_rng(6 + D)
    k = workloads.bf16_round(rng.standard_normal((T, H, D)).astype(np.float32) * 3)
    v = workloads.bf16_round(rng.standard_normal((T, H, D)).astype(np.float32) * 3)
    log(f"cache_write mid-page chunks {mode} D={D}: {T} tokens")
    dtype = "bf16" if mode == "bf16" else "fp8"
    c = kvq.PagedCache(P, H, D, dtype, "per_tensor" if mode == "bf16" else mode)
    c.k_pages.view(torch.uint8).fill_(0x5A)
    c.v_pages.view(torch.uint8).fill_(0x5A)
    kvq.cache_write(c, dev_bf16(k), dev_bf16(v), dev(slots), 0.5, 0.25)
    got = read_pools(c)
    page, off = slots // 16, slots % 16
    if mode == "bf16":
        assert np.array_equal(got["k"][page, :, off], k)
        assert np.array_equal(got["v"][page, :, off], v)
    else:
        want = ocache.new_pools(P, H, D)
        ocache.cache_write(want, k, v, slots, mode, 0.5, 0.25)
        _check_pools(got, want, slots)
    written = np.zeros(P * 16, bool)
    written[slots] = True
    untouched = np.nonzero(~written)[0]
    eb = 2 if mode == "bf16" else 1
    kraw = c.k_pages.view(torch.uint8).cpu().numpy().reshape(P, H, 16, D * eb)
    vraw = c.v_pages.view(torch.uint8).cpu().numpy().reshape(P, H, D, 16, eb)
    assert (kraw[untouched // 16, :, untouched % 16] == 0x5A).all()
    assert (vraw[untouched // 16, :, :, untouched % 16] == 0x5A).all()
