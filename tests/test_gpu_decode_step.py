"""GPU parity: the fused decode step (new-token cache write + decode attention in one
launch) against the two separate calls, and against the float64 oracle.

For each case the cache first holds every token but each sequence's last; path A then
writes the last tokens with kvq.cache_write and runs kvq.decode_attention, path B
runs kvq.decode_step on a second cache with the same history.  The caches must end
byte-identical and the outputs bit-identical (same kernels, same arithmetic), and the
output must meet the oracle's bar.
"""
import numpy as np
import pytest

import workloads
from oracle import attention, cache as ocache

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

from gpu_common import (assert_close_to_oracle, dev, dev_bf16, log,  # noqa: E402
                        oracle_pools, read_pools, write_cache)


@pytest.fixture(scope="module")
def kvq():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import fp8_quantized_paged_amd as k
    return k


def last_rows(case, lens):
    """Row index (into case.k) of position lens[b] - 1 of each sequence, -1 if empty."""
    starts = np.concatenate([[0], np.cumsum(case.seq_lens)[:-1]])
    return np.where(lens > 0, starts + lens - 1, -1)


def new_rows(case, rows):
    """bf16 [B][Hkv][D] rows of the tokens ``rows`` (zeros where rows < 0)."""
    B = len(rows)
    k = np.zeros((B, case.num_kv_heads, case.head_dim), np.float32)
    v = np.zeros_like(k)
    k[rows >= 0] = case.k[rows[rows >= 0]]
    v[rows >= 0] = case.v[rows[rows >= 0]]
    return k, v


def check_step(kvq, case, dtype, mode, q_scale=1.0, k_scale=1.0, v_scale=1.0, pps=0,
               out_dtype="f32", steps=1):
    """History = all tokens but the last ``steps`` of each sequence; then ``steps``
    decode steps, each appending one token per sequence, on both paths."""
    lens = case.seq_lens.astype(np.int64)
    starts = np.concatenate([[0], np.cumsum(lens)[:-1]])
    hist_len = np.maximum(lens - steps, 0)
    hist = np.concatenate([np.arange(s, s + h) for s, h in zip(starts, hist_len)]
                          ).astype(np.int64)
    ca = write_cache(kvq, case, dtype, mode, k_scale, v_scale, rows=hist)
    cb = write_cache(kvq, case, dtype, mode, k_scale, v_scale, rows=hist)
    sc = kvq.Scales(q_scale, k_scale, v_scale, 1.0)
    q = dev_bf16(case.q)
    bt = dev(case.block_table)
    for step in range(steps):
        # the sequences' lengths after this step's token (a sequence already at its
        # full length stores its last token again, which changes nothing)
        cur = np.minimum(hist_len + step + 1, lens).astype(np.int32)
        rows = last_rows(case, cur)
        sel = rows[rows >= 0]
        if len(sel):
            kvq.cache_write(ca, dev_bf16(case.k[sel]), dev_bf16(case.v[sel]),
                            dev(case.slots[sel].astype(np.int64)), k_scale, v_scale)
        maxl = int(cur.max()) if len(cur) else 0
        out_a = kvq.decode_attention(ca, q, bt, dev(cur), maxl, sc, window=case.window,
                                     pages_per_split=pps, out_dtype=out_dtype)
        kn, vn = new_rows(case, rows)
        out_b = kvq.decode_step(cb, q, dev_bf16(kn), dev_bf16(vn), bt, dev(cur), maxl, sc,
                                window=case.window, pages_per_split=pps,
                                out_dtype=out_dtype)
        got_a = out_a.float().cpu().numpy()
        got_b = out_b.float().cpu().numpy()
        assert np.array_equal(got_a, got_b), (
            f"step {step}: outputs differ, max {np.abs(got_a - got_b).max()}")
        pa, pb = read_pools(ca), read_pools(cb)
        for name in pa:
            assert np.array_equal(pa[name], pb[name]), f"step {step}: pool {name} differs"
    # the final state against the oracle: every token written, attention over all
    if dtype == "fp8":
        pools = oracle_pools(case, mode, k_scale, v_scale)
        # written slots only (the oracle's unwritten entries are NaN)
        page, off = case.slots // 16, case.slots % 16
        for name in pa:
            assert np.array_equal(pa[name][page, :, off], pools[name][page, :, off]), (
                f"pool {name} vs oracle")
        kp = ocache.dequantized(pools, "k")
        vp = ocache.dequantized(pools, "v")
        _, qh = ocache.quantize_q(case.q, q_scale)
    else:  # bf16 cache: the raw rows
        kp = np.zeros((case.num_pages, case.num_kv_heads, 16, case.head_dim))
        vp = np.zeros_like(kp)
        page, off = case.slots // 16, case.slots % 16
        kp[page, :, off] = case.k
        vp[page, :, off] = case.v
        qh = case.q
    want = attention.decode(qh, kp, vp, case.block_table, case.seq_lens, case.window)
    return assert_close_to_oracle(got_b, want, "decode step")


@pytest.mark.parametrize("mode", ["per_token_head", "per_tensor"])
@pytest.mark.parametrize("D,Hq,Hkv", [(128, 32, 8), (64, 64, 8), (256, 8, 4), (64, 4, 4),
                                       (128, 128, 8)])
def test_decode_step_matches_separate_calls(kvq, mode, D, Hq, Hkv):
    # ragged lengths: one token, a page boundary either side, several pages
    case = workloads.make_decode_case(300 + D + Hq, [1, 16, 17, 333, 1029], Hq, Hkv, D,
                                      table="perm")
    ks, vs = (1.0, 1.0) if mode == "per_token_head" else (0.05, 0.04)
    log(f"decode step {mode} D={D} Hq={Hq} Hkv={Hkv}")
    check_step(kvq, case, "fp8", mode, q_scale=1.0, k_scale=ks, v_scale=vs)


@pytest.mark.parametrize("pps", [1, 2, 5])
def test_decode_step_small_splits(kvq, pps):
    """Many splits per sequence: the new token lands in the last split only."""
    case = workloads.make_decode_case(411 + pps, [31, 48, 49, 700], 32, 8, 128,
                                      table="perm")
    log(f"decode step pps={pps}")
    check_step(kvq, case, "fp8", "per_token_head", pps=pps, out_dtype="bf16")


def test_decode_step_consecutive(kvq):
    """Several steps in a row, each appending one token per sequence (crossing page
    boundaries), with an empty sequence in the batch."""
    case = workloads.make_decode_case(421, [14, 0, 35, 260, 3], 16, 2, 128, table="perm")
    log("decode step consecutive")
    check_step(kvq, case, "fp8", "per_token_head", steps=6)


@pytest.mark.parametrize("window", [0, 128])
def test_decode_step_bf16_cache(kvq, window):
    """The bf16 skip path: the new row is stored unquantised."""
    case = workloads.make_decode_case(431, [400, 20, 129, 1], 64, 8, 64, table="perm",
                                      window=window)
    log(f"decode step bf16 window {window}")
    check_step(kvq, case, "bf16", "per_token_head", steps=2)


def test_decode_step_window_fp8(kvq):
    case = workloads.make_decode_case(441, [5, 130, 600], 32, 8, 128, table="perm",
                                      window=128)
    log("decode step fp8 window 128")
    check_step(kvq, case, "fp8", "per_token_head", steps=3)


@pytest.mark.parametrize("D,Hq,mode", [(128, 32, "per_token_head"), (64, 64, "per_tensor")])
def test_decode_step_eight_sequences(kvq, D, Hq, mode):
    """8 sequences x 8 KV heads (the Llama- and gpt-oss-shaped head layouts), ragged:
    several splits per sequence, two steps in a row."""
    case = workloads.make_decode_case(431 + D, [1, 16, 17, 333, 1029, 2048, 40, 700], Hq, 8,
                                      D, table="perm")
    ks, vs = (1.0, 1.0) if mode == "per_token_head" else (0.05, 0.04)
    log(f"decode step 8 sequences {mode} D={D} Hq={Hq}")
    check_step(kvq, case, "fp8", mode, k_scale=ks, v_scale=vs, steps=2)
