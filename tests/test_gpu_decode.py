"""GPU parity: split-K paged decode attention against the float64 oracle."""
import math

import numpy as np
import pytest

import workloads
from oracle import attention, cache as ocache

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

from gpu_common import (assert_close_to_oracle, check_bf16_bar, dev, dev_bf16,  # noqa: E402
                        log, oracle_pools, oracle_pools_for_heads, raw_pools_for_heads,
                        write_cache)


@pytest.fixture(scope="module")
def kvq():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import fp8_quantized_paged_amd as k
    return k


def run_decode(kvq, c, case, mode, q_scale=1.0, k_scale=1.0, v_scale=1.0, window=None,
               pps=0, out_dtype="f32"):
    window = case.window if window is None else window
    sc = kvq.Scales(q_scale, k_scale, v_scale, 1.0)
    out = kvq.decode_attention(c, dev_bf16(case.q), dev(case.block_table),
                               dev(case.seq_lens), int(case.seq_lens.max()), sc,
                               window=window, pages_per_split=pps, out_dtype=out_dtype)
    return out.float().cpu().numpy()


def oracle_decode(case, mode, q_scale=1.0, k_scale=1.0, v_scale=1.0, window=None,
                  heads=None):
    window = case.window if window is None else window
    pools = oracle_pools(case, mode, k_scale, v_scale)
    kp = ocache.dequantized(pools, "k")
    vp = ocache.dequantized(pools, "v")
    _, qh = ocache.quantize_q(case.q, q_scale)
    return attention.decode(qh, kp, vp, case.block_table, case.seq_lens, window,
                            heads=heads)


@pytest.mark.parametrize("mode", ["per_tensor", "per_token_head"])
def test_tiny_decode(kvq, mode):
    case = workloads.tiny_decode()
    log(f"decode tiny {mode}")
    c = write_cache(kvq, case, "fp8", mode)
    got = run_decode(kvq, c, case, mode)
    want = oracle_decode(case, mode)
    assert_close_to_oracle(got, want, f"tiny {mode}")
    gotb = run_decode(kvq, c, case, mode, out_dtype="bf16")
    assert_close_to_oracle(gotb, want, f"tiny {mode} bf16 out")
    kp, vp = raw_pools_for_heads(case, 0, [0])
    want_bf16 = attention.decode(case.q, kp, vp, case.block_table, case.seq_lens)
    check_bf16_bar(got, want_bf16, want, f"tiny {mode}")


# group sizes 1 .. 16 at every head_dim: both kernel forms (vector ALU for small
# groups, matrix cores for groups of 8 and 16)
@pytest.mark.parametrize("D,Hq,Hkv", [(64, 4, 4), (64, 16, 2), (128, 32, 8), (128, 16, 1),
                                       (256, 8, 4), (64, 64, 8), (128, 8, 4), (128, 64, 8),
                                       (64, 32, 2), (256, 32, 2), (256, 16, 2)])
def test_ragged_batch(kvq, D, Hq, Hkv):
    lens = [0, 1, 15, 16, 17, 100, 1000, 33]
    case = workloads.make_decode_case(50 + D + Hq, lens, Hq, Hkv, D, table="perm",
                                      outliers=4, extra_pages=3)
    for mode, qs, ks, vs in (("per_token_head", 1.0, 1.0, 1.0),
                             ("per_tensor", 0.75, 1.0, 1.0), ("per_tensor", 1.0, 0.05, 0.1)):
        log(f"decode ragged D={D} Hq={Hq} Hkv={Hkv} {mode} q={qs} k={ks} v={vs}")
        c = write_cache(kvq, case, "fp8", mode, ks, vs)
        got = run_decode(kvq, c, case, mode, qs, ks, vs)
        want = oracle_decode(case, mode, qs, ks, vs)
        assert_close_to_oracle(got, want, f"ragged D={D} {mode}")
        assert not got[0].any()   # empty sequence


@pytest.mark.parametrize("window", [1, 5, 16, 17, 128, 5000])
def test_sliding_window_fp8(kvq, window):
    case = workloads.make_decode_case(60, [300, 129, 2, 1000], 16, 2, 64, table="perm")
    log(f"decode window {window}")
    c = write_cache(kvq, case, "fp8", "per_token_head")
    got = run_decode(kvq, c, case, "per_token_head", window=window)
    want = oracle_decode(case, "per_token_head", window=window)
    assert_close_to_oracle(got, want, f"window {window}")


@pytest.mark.parametrize("window", [0, 128])
def test_bf16_cache_skip_path(kvq, window):
    """Sliding-window layers keep a bf16 cache: attention over the raw bf16 values."""
    case = workloads.make_decode_case(61, [400, 20, 129], 64, 8, 64, table="perm")
    log(f"decode bf16 window {window}")
    c = write_cache(kvq, case, "bf16")
    got = run_decode(kvq, c, case, None, window=window)
    kp = np.zeros((case.num_pages, 8, 16, 64))
    vp = np.zeros_like(kp)
    page, off = case.slots // 16, case.slots % 16
    kp[page, :, off] = case.k
    vp[page, :, off] = case.v
    want = attention.decode(case.q, kp, vp, case.block_table, case.seq_lens, window)
    assert_close_to_oracle(got, want, "bf16 cache")


def test_split_count_invariance_and_determinism(kvq):
    case = workloads.make_decode_case(62, [2000, 777], 32, 8, 128, table="perm", outliers=4)
    c = write_cache(kvq, case, "fp8", "per_token_head")
    base = run_decode(kvq, c, case, "per_token_head", pps=4)
    # Between split counts the float32 summation order changes, and so does each
    # wave's softmax reference maximum, against which the PV weights are rounded to
    # f16 (unit roundoff 2^-11).  Two such roundings of the weights of
    # o = sum_j w_j v_j / sum_j w_j differ by at most 2 * 2^-11 * sum_j w_j |v_j| /
    # sum_j w_j, i.e. twice the attention output over |v|, which the oracle gives.
    pools = oracle_pools(case, "per_token_head")
    _, qh = ocache.quantize_q(case.q, 1.0)
    abs_out = attention.decode(qh, ocache.dequantized(pools, "k"),
                               np.abs(ocache.dequantized(pools, "v")), case.block_table,
                               case.seq_lens)
    bound = 1e-5 + 1e-5 * np.abs(base) + 2.0 ** -10 * abs_out
    for pps in (1, 7, 16, 64, 0):
        other = run_decode(kvq, c, case, "per_token_head", pps=pps)
        assert np.all(np.abs(other - base) <= bound), pps
    again = [run_decode(kvq, c, case, "per_token_head", pps=16) for _ in range(5)]
    for a in again[1:]:
        assert np.array_equal(a, again[0])


def test_workspace_reuse_across_calls(kvq):
    """One workspace serves consecutive calls with different inputs, batch sizes and
    split counts: the counter prefix sits at a fixed place, so a small call's partials
    never land on a larger call's counters, and every call leaves the counters zero."""
    a = workloads.make_decode_case(63, [3000, 900, 0, 40], 32, 8, 128, table="perm")
    b = workloads.make_decode_case(64, [2500, 17, 1300, 4000], 32, 8, 128, table="perm")
    # 16 sequences, then one long sequence with many splits (its partials start right
    # after the counter prefix, where a layout sized by the batch would put counters
    # 16 .. 127 of the 16-sequence call), then the 16 sequences again
    many = workloads.make_decode_case(65, list(range(100, 100 + 16 * 300, 300)), 32, 8, 128,
                                      table="perm")
    one = workloads.make_decode_case(66, [6000], 32, 8, 128, table="perm")
    caches = {id(x): write_cache(kvq, x, "fp8", "per_token_head") for x in (a, b, many, one)}
    need = max(kvq.decode_workspace_bytes(caches[id(x)], len(x.seq_lens), 32,
                                          int(x.seq_lens.max()), 0, 4)
               for x in (a, b, many, one))
    ws = torch.zeros(need, dtype=torch.uint8, device="cuda")
    sc = kvq.Scales(1.0, 1.0, 1.0, 1.0)

    def call(case):
        return kvq.decode_attention(caches[id(case)], dev_bf16(case.q),
                                    dev(case.block_table), dev(case.seq_lens),
                                    int(case.seq_lens.max()), sc, pages_per_split=4,
                                    out_dtype="f32", workspace=ws).cpu().numpy()
    want = {id(x): oracle_decode(x, "per_token_head") for x in (a, b, many, one)}
    for _ in range(2):
        for x, name in ((a, "a"), (b, "b"), (many, "16 seqs"), (one, "1 seq"),
                        (many, "16 seqs again"), (a, "a again")):
            assert_close_to_oracle(call(x), want[id(x)], f"reuse {name}")
    assert not ws[:kvq.DECODE_COUNTER_BYTES].any()   # counters back at zero


def test_lengths_above_max_seq_len_stay_in_bounds(kvq):
    """A device length above the call's max_seq_len (a precondition the host cannot
    check) is read only up to max_seq_len: the other sequences stay exact, the
    counters return to zero and a following call on the same workspace is exact."""
    case = workloads.make_decode_case(67, [700, 300, 1000], 32, 8, 128, table="perm")
    c = write_cache(kvq, case, "fp8", "per_token_head")
    ws = kvq.decode_workspace(c, 3, 32, 1000, 0, 4)
    sc = kvq.Scales(1.0, 1.0, 1.0, 1.0)
    # max_seq_len 600 but sequence 2 claims 1000 tokens
    got = kvq.decode_attention(c, dev_bf16(case.q), dev(case.block_table),
                               dev(case.seq_lens), 600, sc, pages_per_split=4,
                               out_dtype="f32", workspace=ws).cpu().numpy()
    want = oracle_decode(case, "per_token_head")
    assert_close_to_oracle(got[1], want[1], "in-range sequence beside a long one")
    assert np.isfinite(got).all()
    assert not ws[:kvq.DECODE_COUNTER_BYTES].any()
    full = kvq.decode_attention(c, dev_bf16(case.q), dev(case.block_table),
                                dev(case.seq_lens), 1000, sc, pages_per_split=4,
                                out_dtype="f32", workspace=ws).cpu().numpy()
    assert_close_to_oracle(full, want, "the next call on the same workspace")


def test_llama8b_decode_sampled(kvq):
    """Llama-3.1-8B-shaped decode layer at full size (8 x 20,000 tokens, seeded
    permutation block table, outliers, per-token-head scales), in the launch
    configuration the benchmark times; sampled (sequence, head) outputs against the
    oracle."""
    case = workloads.llama8b_decode()
    log("decode llama8b: writing cache")
    c = write_cache(kvq, case, "fp8", "per_token_head", chunk=1 << 24)
    got = run_decode(kvq, c, case, "per_token_head", out_dtype="bf16")
    rng = np.random.default_rng(1)
    picks = [(int(b), int(g)) for b, g in zip(rng.integers(0, 8, 6), rng.integers(0, 8, 6))]
    _, qh = ocache.quantize_q(case.q, 1.0)
    for b, g in picks:
        log(f"  oracle seq {b} kv head {g}")
        kp, vp = oracle_pools_for_heads(case, b, [g], "per_token_head")
        heads = [(b, h) for h in range(g * 4, g * 4 + 4)]
        want = attention.decode(qh, kp, vp, case.block_table, case.seq_lens, 0,
                                heads=heads)
        for _, h in heads:
            assert_close_to_oracle(got[b, h], want[b, h], f"llama8b b={b} h={h}")
        # the bf16-cache result: the outlier channels (x20) make K's quantisation move
        # the scores enough that the oracle's own exact result misses the 6e-2 bar on a
        # few percent of elements, so the device is held to the oracle's distance
        rk, rv = raw_pools_for_heads(case, b, [g])
        want_bf16 = attention.decode(case.q, rk, rv, case.block_table, case.seq_lens, 0,
                                     heads=heads)
        hs = [h for _, h in heads]
        check_bf16_bar(got[b, hs], want_bf16[b, hs], want[b, hs], f"llama8b b={b} g={g}",
                       require=False)


def test_long_context_planted_key(kvq):
    """131,072-token accumulation stress: sampled KV heads match the oracle and every
    aligned head retrieves the planted V row."""
    case = workloads.long_context_decode()
    log("decode 131k: writing cache")
    c = write_cache(kvq, case, "fp8", "per_tensor", chunk=1 << 24)
    got = run_decode(kvq, c, case, "per_tensor")
    _, qh = ocache.quantize_q(case.q, 1.0)
    for g in (0, 5):
        log(f"  oracle kv head {g}")
        kp, vp = oracle_pools_for_heads(case, 0, [g], "per_tensor")
        heads = [(0, h) for h in range(g * 4, g * 4 + 4)]
        want = attention.decode(qh, kp, vp, case.block_table, case.seq_lens, 0,
                                heads=heads)
        for _, h in heads:
            assert_close_to_oracle(got[0, h], want[0, h], f"131k h={h}")
        rk, rv = raw_pools_for_heads(case, 0, [g])
        want_bf16 = attention.decode(case.q, rk, rv, case.block_table, case.seq_lens, 0,
                                     heads=heads)
        hs = [h for _, h in heads]
        check_bf16_bar(got[0, hs], want_bf16[0, hs], want[0, hs], f"131k g={g}")
    pos = case.meta["planted_pos"]
    for g in range(8):
        h = g * 4
        o = got[0, h]
        v = case.v[:, g].astype(np.float64)
        cos = v @ o / (np.linalg.norm(v, axis=1) * np.linalg.norm(o))
        assert int(np.argmax(cos)) == pos, g
        assert cos[pos] > 0.9, (g, cos[pos])


@pytest.mark.parametrize("layer", [0, 1])
def test_gptoss_hybrid_layers_sampled(kvq, layer):
    """gpt-oss-20b-shaped layers at full size: an fp8 full-attention layer and a bf16
    sliding-window-128 layer (the skip path); sampled sequences against the oracle."""
    case = workloads.gptoss_hybrid_layer(layer)
    dtype = kvq.layer_kv_dtype(case.window, kvq.SKIP_SLIDING_WINDOW)
    assert dtype == ("fp8" if layer % 2 == 0 else "bf16")
    log(f"decode gpt-oss layer {layer} ({dtype})")
    c = write_cache(kvq, case, dtype, "per_tensor", chunk=1 << 24)
    got = run_decode(kvq, c, case, "per_tensor")
    for b in (0, 5):
        heads = [(b, h) for h in range(64)]
        if dtype == "fp8":
            kp, vp = oracle_pools_for_heads(case, b, range(8), "per_tensor")
            _, qh = ocache.quantize_q(case.q, 1.0)
        else:
            sel = np.nonzero(case.token_seq == b)[0]
            kp = np.zeros((case.num_pages, 8, 16, 64))
            vp = np.zeros_like(kp)
            page, off = case.slots[sel] // 16, case.slots[sel] % 16
            kp[page, :, off] = case.k[sel]
            vp[page, :, off] = case.v[sel]
            qh = case.q
        want = attention.decode(qh, kp, vp, case.block_table, case.seq_lens,
                                case.window, heads=heads)
        assert_close_to_oracle(got[b], want[b], f"gpt-oss layer {layer} b={b}")
        rk, rv = raw_pools_for_heads(case, b, range(8))
        want_bf16 = attention.decode(case.q, rk, rv, case.block_table, case.seq_lens,
                                     case.window, heads=heads)
        check_bf16_bar(got[b], want_bf16[b], want[b], f"gpt-oss layer {layer} b={b}")
