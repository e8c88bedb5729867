"""GPU parity: chunked FP8 prefill attention (FP8 matrix cores) against the float64
oracle computed from the same dequantised cache and quantised queries.

The device rounds the softmax weights to e4m3 before the P.V product and normalises by
the sum of the same rounded weights, so its output is the exact attention with every
weight w_j carrying a relative error d_j, renormalised.  The bound on |d_j| follows
from the kernel's stated invariants (prefill_kernel.h, "Softmax"): the weight handed to
the rounding is P_j = 2^(x_j - m) f_j, where x_j is the key's log2-domain score, the
reference m is at most the row's largest score minus 4 (so P_j >= 2^(gap_j + 4) f_j,
gap_j = x_j - max x <= 0), and f_j = v_scale_j / (v_ref prob_scale) with v_ref at most
the largest V scale of the sequence's KV head (per-tensor and per-KV-head modes:
f_j = 1 / prob_scale).  Round-to-nearest e4m3 errs by at most 2^-4 P (normal values,
3 mantissa bits) or 2^-10 (the subnormal grid 2^-9, values below 2^-6; below 2^-10
the weight may flush to zero), and a non-negative weight cannot err by more than
itself: |d_j| <= min(1, max(2^-4, 2^-10 / (2^(gap_j + 4) f_j))).  The oracle turns
those per-key bounds into the largest move of the renormalised mean (attend_rows'
weight_error), which the tests add to the plain 5e-3 + 2e-2 |O| bar.  The full-size
head_dim-256 workload and the 131,072-key stress test are held to the plain bar.
"""
import ctypes

import numpy as np
import pytest

import workloads
from oracle import attention, cache as ocache

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

from gpu_common import (ATOL, RTOL, assert_close_to_oracle, check_bf16_bar,  # noqa: E402
                        dev, dev_bf16, log, oracle_pools, raw_pools_for_heads, write_cache)


@pytest.fixture(scope="module")
def kvq():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import fp8_quantized_paged_amd as k
    return k


# The kernel's reference puts a row's largest weight at 2^REF_TOP or above.
REF_TOP = 4.0


def p_rounding_error(case, pools, mode, prob_scale=1.0):
    """Per (sequence b, KV head g): the function (gap, j) -> bound on the relative
    error of key j's rounded weight (module docstring)."""
    def for_head(b, g):
        if mode == "per_token_head":
            sel = np.nonzero(case.token_seq == b)[0]
            page, off = case.slots[sel] // 16, case.slots[sel] % 16
            vs = np.zeros(int(case.seq_lens[b]))
            vs[case.token_pos[sel]] = pools["v_scales"][page, g, off]
            f = vs / (vs.max() * prob_scale)
        else:
            f = np.full(int(case.seq_lens[b]), 1.0 / prob_scale)

        def err(gap, js):
            low = np.exp2(gap + REF_TOP) * f[js]
            with np.errstate(divide="ignore"):
                return np.minimum(1.0, np.maximum(2.0 ** -4, 2.0 ** -10 / low))
        return err
    return for_head


def assert_close_with_p_rounding(got, want, bound, what=""):
    err = np.abs(got - want)
    lim = ATOL + RTOL * np.abs(want) + bound
    bad = err > lim
    if bad.any():
        i = np.unravel_index(np.argmax(err - lim), err.shape)
        raise AssertionError(
            f"{what}: {int(bad.sum())}/{bad.size} outside the bound; worst at {i}: got "
            f"{got[i]!r} want {want[i]!r} rounding bound {bound[i]!r}")


def run_prefill(kvq, c, case, q_scale=1.0, k_scale=1.0, v_scale=1.0, prob_scale=1.0,
                causal=True, window=0, out_dtype="f32", accumulation=None, split=True):
    sc = kvq.Scales(q_scale, k_scale, v_scale, prob_scale)
    q_lens = np.diff(case.cu_q_lens)
    out = kvq.prefill_attention(c, dev_bf16(case.q), dev(case.cu_q_lens),
                                dev(case.block_table), dev(case.seq_lens),
                                int(q_lens.max()), sc, causal=causal, window=window,
                                out_dtype=out_dtype, accumulation=accumulation,
                                split=split)
    return out.float().cpu().numpy()


def oracle_prefill(case, mode, q_scale=1.0, k_scale=1.0, v_scale=1.0, causal=True,
                   window=0, rows=None, p_bound=False, prob_scale=1.0):
    """The oracle's attention; with p_bound also the rounding bound of every output
    element (module docstring)."""
    pools = oracle_pools(case, mode, k_scale, v_scale)
    _, qh = ocache.quantize_q(case.q, q_scale)
    we = p_rounding_error(case, pools, mode, prob_scale) if p_bound else None
    return attention.prefill(qh, case.cu_q_lens, ocache.dequantized(pools, "k"),
                             ocache.dequantized(pools, "v"), case.block_table,
                             case.seq_lens, causal, window, rows=rows, weight_error=we)


@pytest.mark.parametrize("D,Hq,Hkv", [(256, 8, 4), (128, 32, 8), (64, 16, 2),
                                       (128, 16, 1), (256, 4, 4)])
@pytest.mark.parametrize("mode", ["per_token_head", "per_tensor"])
def test_prefill_ragged(kvq, D, Hq, Hkv, mode):
    # several sequences, contexts and chunk lengths that are not tile multiples
    ctx, new = [0, 37, 300, 1000], [70, 1, 150, 129]
    case = workloads.make_prefill_case(200 + D + Hq, ctx, new, Hq, Hkv, D, table="perm",
                                       extra_pages=5)
    ks, vs = (1.0, 1.0) if mode == "per_token_head" else (0.5, 0.25)
    log(f"prefill ragged D={D} Hq={Hq} Hkv={Hkv} {mode}")
    c = write_cache(kvq, case, "fp8", mode, ks, vs)
    got = run_prefill(kvq, c, case, k_scale=ks, v_scale=vs)
    want, bound = oracle_prefill(case, mode, k_scale=ks, v_scale=vs, p_bound=True)
    assert_close_with_p_rounding(got, want, bound, f"prefill D={D} {mode}")
    gotb = run_prefill(kvq, c, case, k_scale=ks, v_scale=vs, out_dtype="bf16")
    assert_close_with_p_rounding(gotb, want, bound, f"prefill D={D} {mode} bf16 out")


@pytest.mark.parametrize("D,Hq,Hkv,mode", [(256, 8, 4, "per_token_head"),
                                            (128, 32, 8, "per_tensor"),
                                            (64, 16, 2, "per_token_head")])
def test_prefill_ragged_valu_add(kvq, D, Hq, Hkv, mode):
    """The explicit-flush form of level 2 (each 64-key chunk into a zeroed accumulator,
    float32 vector adds) on the ragged shapes."""
    ctx, new = [0, 37, 300, 1000], [70, 1, 150, 129]
    case = workloads.make_prefill_case(200 + D + Hq, ctx, new, Hq, Hkv, D, table="perm",
                                       extra_pages=5)
    ks, vs = (1.0, 1.0) if mode == "per_token_head" else (0.5, 0.25)
    log(f"prefill ragged valu_add D={D} Hq={Hq} Hkv={Hkv} {mode}")
    c = write_cache(kvq, case, "fp8", mode, ks, vs)
    got = run_prefill(kvq, c, case, k_scale=ks, v_scale=vs, accumulation="valu_add")
    want, bound = oracle_prefill(case, mode, k_scale=ks, v_scale=vs, p_bound=True)
    assert_close_with_p_rounding(got, want, bound, f"prefill valu_add D={D} {mode}")


def test_long_context_prefill_planted_key(kvq):
    """Two-level accumulation past 100k keys on the FP8 matrix cores: 128 new queries at
    the end of a 131,072-token sequence (per-token-head scales, a planted key in the
    first 16,384 positions).  Every output element of every row and head, in both
    level-2 forms, is held to the plain 5e-3 + 2e-2 |O| bar against the float64
    oracle; the heads aligned with the planted key retrieve its V row; and the two
    forms agree to within what float32 accumulation of the 2,048 chunk sums allows
    (each form within 2,048 * 2^-24 * max_j |v_j| of the exact sum), which a
    reduced-precision running accumulator would exceed by orders of magnitude."""
    case = workloads.long_context_prefill()
    pos = case.meta["planted_pos"]
    log(f"prefill 131k: writing cache (planted key at {pos})")
    c = write_cache(kvq, case, "fp8", "per_token_head", chunk=1 << 24)
    got = {}
    for acc in ("mfma_chain", "valu_add"):
        log(f"prefill 131k: device run, {acc}")
        got[acc] = run_prefill(kvq, c, case, accumulation=acc)
    log("prefill 131k: oracle (128 rows x 32 heads x 131,072 keys)")
    pools = oracle_pools(case, "per_token_head")
    _, qh = ocache.quantize_q(case.q, 1.0)
    vp = ocache.dequantized(pools, "v")
    want = attention.prefill(qh, case.cu_q_lens, ocache.dequantized(pools, "k"), vp,
                             case.block_table, case.seq_lens, True, 0)
    L = int(case.seq_lens[0])
    G = 4
    for acc, o in got.items():
        assert np.isfinite(o).all(), acc
        err = assert_close_to_oracle(o, want, f"131k prefill {acc}")
        log(f"  {acc}: max abs err {err:.3g} (max |O| {np.abs(want).max():.3g})")
        for g in range(8):   # the last row's first head of each group is aligned
            v = case.v[:L, g].astype(np.float64)
            out = o[-1, g * G]
            cos = v @ out / (np.linalg.norm(v, axis=1) * np.linalg.norm(out))
            assert int(np.argmax(cos)) == pos and cos[pos] > 0.9, (acc, g, cos[pos])
    vmax = np.abs(attention.gather(vp, case.block_table[0], L)).max(axis=0)  # [Hkv][D]
    lim = 2.0 * 2048 * 2.0 ** -24 * np.repeat(vmax, G, axis=0)[None]
    diff = np.abs(got["mfma_chain"] - got["valu_add"])
    log(f"  chain vs valu_add: max diff {diff.max():.3g}, limit {lim.min():.3g}..")
    assert np.all(diff <= lim)


@pytest.mark.parametrize("window", [1, 17, 100])
def test_prefill_sliding_window(kvq, window):
    case = workloads.make_prefill_case(231, [500, 64], [200, 90], 8, 2, 128, table="perm")
    log(f"prefill window {window}")
    c = write_cache(kvq, case, "fp8", "per_token_head")
    got = run_prefill(kvq, c, case, window=window)
    want, bound = oracle_prefill(case, "per_token_head", window=window, p_bound=True)
    assert_close_with_p_rounding(got, want, bound, f"prefill window {window}")


def test_prefill_non_causal_and_scales(kvq):
    case = workloads.make_prefill_case(232, [129, 0], [64, 33], 16, 4, 256, table="perm")
    log("prefill non-causal, q_scale 0.5, prob_scale 2")
    c = write_cache(kvq, case, "fp8", "per_tensor", 0.75, 1.5)
    got = run_prefill(kvq, c, case, q_scale=0.5, k_scale=0.75, v_scale=1.5,
                      prob_scale=2.0, causal=False)
    want, bound = oracle_prefill(case, "per_tensor", q_scale=0.5, k_scale=0.75,
                                 v_scale=1.5, causal=False, p_bound=True, prob_scale=2.0)
    assert_close_with_p_rounding(got, want, bound, "prefill non-causal")


def test_prefill_last_row_matches_decode(kvq):
    """The last query row of a prefill chunk is the decode query of that sequence."""
    case = workloads.make_prefill_case(233, [777], [50], 32, 8, 128, table="perm")
    c = write_cache(kvq, case, "fp8", "per_token_head")
    got = run_prefill(kvq, c, case)
    q_last = case.q[-1:]
    dec = kvq.decode_attention(c, dev_bf16(q_last), dev(case.block_table),
                               dev(case.seq_lens), int(case.seq_lens[0]),
                               kvq.Scales(1.0, 1.0, 1.0, 1.0),
                               out_dtype="f32").cpu().numpy()
    want, bound = oracle_prefill(case, "per_token_head", p_bound=True)
    assert_close_to_oracle(dec, want[-1:], "decode of the last row")
    assert_close_with_p_rounding(got[-1:], want[-1:], bound[-1:], "prefill last row")


def test_unwritten_slots_do_not_leak(kvq):
    """Slots past each sequence's end hold NaN codes and NaN scales; neither kernel
    may let them reach the output."""
    case = workloads.make_prefill_case(234, [40, 3], [9, 20], 8, 4, 256, table="perm",
                                       extra_pages=2)
    c = kvq.PagedCache(case.num_pages, case.num_kv_heads, case.head_dim, "fp8",
                       "per_token_head")
    c.k_pages.fill_(0x7F)
    c.v_pages.fill_(0xFF)
    c.k_scales.fill_(float("nan"))
    c.v_scales.fill_(float("nan"))
    kvq.cache_write(c, dev_bf16(case.k), dev_bf16(case.v),
                    dev(case.slots.astype(np.int64)))
    got = run_prefill(kvq, c, case)
    want, bound = oracle_prefill(case, "per_token_head", p_bound=True)
    assert np.isfinite(got).all()
    assert_close_with_p_rounding(got, want, bound, "prefill with NaN-filled free slots")
    last = case.cu_q_lens[1:] - 1
    dec = kvq.decode_attention(c, dev_bf16(case.q[last]), dev(case.block_table),
                               dev(case.seq_lens), int(case.seq_lens.max()),
                               kvq.Scales(1.0, 1.0, 1.0, 1.0),
                               out_dtype="f32").cpu().numpy()
    assert np.isfinite(dec).all()
    assert_close_to_oracle(dec, want[last], "decode with NaN-filled free slots")


def test_hd256_prefill_sampled(kvq):
    """The head_dim-256 chunked-prefill workload at full size (8,192 new queries on a
    32,768-token cache, 8/4 heads, per-token-head scales), checked on sampled rows:
    the first and last 64 query positions and 64 seeded ones in between."""
    case = workloads.hd256_prefill()
    log("hd256 prefill: writing cache")
    c = write_cache(kvq, case, "fp8", "per_token_head")
    log("hd256 prefill: device run")
    got = run_prefill(kvq, c, case)
    n = int(case.cu_q_lens[1])
    rng = np.random.default_rng(7)
    rows = np.unique(np.concatenate([np.arange(64), np.arange(n - 64, n),
                                     rng.choice(n, 64, replace=False)]))
    log(f"hd256 prefill: oracle on {len(rows)} rows")
    want = oracle_prefill(case, "per_token_head", rows=rows)
    assert np.isfinite(got).all()
    assert_close_to_oracle(got[rows], want[rows], "hd256 prefill sampled rows")
    rk, rv = raw_pools_for_heads(case, 0, range(case.num_kv_heads))
    want_bf16 = attention.prefill(case.q, case.cu_q_lens, rk, rv, case.block_table,
                                  case.seq_lens, True, 0, rows=rows)
    check_bf16_bar(got[rows], want_bf16[rows], want[rows], "hd256 prefill sampled rows")


# bf16 weights in P . V: relative rounding error <= 2^-9, renormalised
P_ROUND_BF16 = 2.0 ** -9 / (1.0 - 2.0 ** -9)


@pytest.mark.parametrize("D,Hq,Hkv", [(64, 64, 8), (128, 16, 2), (256, 8, 4)])
@pytest.mark.parametrize("window", [0, 128])
def test_prefill_bf16_cache(kvq, D, Hq, Hkv, window):
    """Sliding-window layers keep a bf16 cache ("Hybrid attention and layer
    skipping"): prefill over the raw bf16 values, causal, with and without a window."""
    ctx, new = [0, 37, 300, 1000], [70, 1, 150, 200]
    case = workloads.make_prefill_case(260 + D + window, ctx, new, Hq, Hkv, D,
                                       table="perm", extra_pages=3)
    log(f"prefill bf16 cache D={D} Hq={Hq} Hkv={Hkv} window={window}")
    c = write_cache(kvq, case, "bf16")
    got = run_prefill(kvq, c, case, window=window)
    kp = np.zeros((case.num_pages, Hkv, 16, D))
    vp = np.zeros_like(kp)
    page, off = case.slots // 16, case.slots % 16
    kp[page, :, off] = case.k
    vp[page, :, off] = case.v
    want, spread = attention.prefill(case.q.astype(np.float64), case.cu_q_lens, kp, vp,
                                     case.block_table, case.seq_lens, True, window,
                                     spread=True)
    err = np.abs(got - want)
    bound = ATOL + RTOL * np.abs(want) + P_ROUND_BF16 * spread
    assert (err <= bound).all(), f"max excess {np.max(err - bound):.3g}"


@pytest.mark.parametrize("D,Hq,Hkv", [(128, 32, 8), (64, 16, 1), (256, 8, 4)])
@pytest.mark.parametrize("mode", ["per_token_head", "per_tensor"])
def test_prefill_key_splits(kvq, D, Hq, Hkv, mode):
    """Short query chunks on a long context: the launch splits each workgroup's keys
    (16 new tokens on 20,000 cached beside 3 on 5: 32-64 splits, most of them empty for
    the short sequence) and merges the partial results; the same call without the
    split, both against the oracle, f32 and bf16 output."""
    case = workloads.make_prefill_case(900 + D + Hq, [20000, 5], [16, 3], Hq, Hkv, D,
                                       table="perm")
    ks, vs = (1.0, 1.0) if mode == "per_token_head" else (0.5, 0.25)
    c = write_cache(kvq, case, "fp8", mode, ks, vs)
    want, bound = oracle_prefill(case, mode, k_scale=ks, v_scale=vs, p_bound=True)
    nb = kvq.binding._lib.kvq_prefill_workspace_bytes(ctypes.byref(c.desc()), 2, Hq, 16)
    assert nb > 0, "this shape should split"
    for split in (True, False):
        log(f"prefill key splits D={D} Hq={Hq} Hkv={Hkv} {mode} split={split}")
        got = run_prefill(kvq, c, case, k_scale=ks, v_scale=vs, split=split)
        assert_close_with_p_rounding(got, want, bound, f"split={split} D={D} {mode}")
    gotb = run_prefill(kvq, c, case, k_scale=ks, v_scale=vs, out_dtype="bf16")
    assert_close_with_p_rounding(gotb, want, bound, f"split D={D} {mode} bf16 out")


def test_prefill_key_splits_window_and_workspace(kvq):
    """A sliding window with key splits (most splits hold none of a row's keys), and a
    workspace one byte short of what the library asks for: INVALID_ARG, nothing run."""
    case = workloads.make_prefill_case(931, [12000], [40], 32, 8, 128, table="perm")
    c = write_cache(kvq, case, "fp8", "per_token_head")
    log("prefill key splits, window 100")
    got = run_prefill(kvq, c, case, window=100)
    want, bound = oracle_prefill(case, "per_token_head", window=100, p_bound=True)
    assert_close_with_p_rounding(got, want, bound, "split window 100")
    nb = kvq.binding._lib.kvq_prefill_workspace_bytes(ctypes.byref(c.desc()), 1, 32, 40)
    assert nb > 0
    short = torch.empty(nb - 1, dtype=torch.uint8, device="cuda")
    with pytest.raises(Exception, match="workspace"):
        kvq.prefill_attention(c, dev_bf16(case.q), dev(case.cu_q_lens),
                              dev(case.block_table), dev(case.seq_lens), 40,
                              kvq.Scales(1.0, 1.0, 1.0, 1.0), workspace=short)
