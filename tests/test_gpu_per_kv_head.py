"""GPU parity: per-KV-head scale arrays ("vLLM FP8 KV-Cache and Attention Quantization
Update", section "Kernel and fusion optimizations": one scale per KV head) through the
cache write, decode (both kernel forms), the decode step and prefill, against the
oracle with the same per-head scales."""
import numpy as np
import pytest

import workloads
from oracle import attention, cache as ocache

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

from gpu_common import (assert_close_to_oracle, dev, dev_bf16, log,  # noqa: E402
                        oracle_pools, read_pools, write_cache)
from test_gpu_prefill import (assert_close_with_p_rounding, oracle_prefill,  # noqa: E402
                              run_prefill)


@pytest.fixture(scope="module")
def kvq():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import fp8_quantized_paged_amd as k
    return k


def head_scales(seed, n):
    """Per-head scales spanning ~30x (some heads saturate their outlier channels)."""
    rng = np.random.default_rng(seed)
    return (0.004 * 2.0 ** rng.uniform(0, 5, n)).astype(np.float32)


def test_cache_write_codes_bit_exact(kvq):
    case = workloads.make_decode_case(701, [33, 1, 250], 16, 4, 128, table="perm",
                                      outliers=2)
    ks, vs = head_scales(1, 4), head_scales(2, 4)
    log("per-KV-head cache write")
    c = write_cache(kvq, case, "fp8", "per_kv_head", ks, vs)
    got = read_pools(c)
    want = oracle_pools(case, "per_kv_head", ks, vs)
    page, off = case.slots // 16, case.slots % 16
    for name in ("k_codes", "v_codes"):
        assert np.array_equal(got[name][page, :, off], want[name][page, :, off]), name


@pytest.mark.parametrize("D,Hq,Hkv", [(128, 32, 8), (64, 64, 8), (128, 64, 8), (256, 8, 4)])
def test_decode(kvq, D, Hq, Hkv):
    case = workloads.make_decode_case(710 + D + Hq, [0, 1, 17, 300, 1500], Hq, Hkv, D,
                                      table="perm", outliers=2)
    ks, vs = head_scales(D + Hq, Hkv), head_scales(D + Hq + 1, Hkv)
    qs = 0.75
    log(f"per-KV-head decode D={D} Hq={Hq} Hkv={Hkv}")
    c = write_cache(kvq, case, "fp8", "per_kv_head", ks, vs)
    out = kvq.decode_attention(c, dev_bf16(case.q), dev(case.block_table),
                               dev(case.seq_lens), int(case.seq_lens.max()),
                               kvq.Scales(qs, 1.0, 1.0, 1.0), out_dtype="f32")
    got = out.cpu().numpy()
    pools = oracle_pools(case, "per_kv_head", ks, vs)
    _, qh = ocache.quantize_q(case.q, qs)
    want = attention.decode(qh, ocache.dequantized(pools, "k"),
                            ocache.dequantized(pools, "v"), case.block_table,
                            case.seq_lens)
    assert_close_to_oracle(got, want, f"per-KV-head decode D={D}")
    assert not got[0].any()


def test_decode_step_matches_separate_calls(kvq):
    """The fused step stores the new rows with the head's scale, as the cache write."""
    case = workloads.make_decode_case(730, [5, 16, 17, 900], 64, 8, 64, table="perm")
    ks, vs = head_scales(31, 8), head_scales(32, 8)
    lens = case.seq_lens.astype(np.int64)
    starts = np.concatenate([[0], np.cumsum(lens)[:-1]])
    last = starts + lens - 1
    hist = np.setdiff1d(np.arange(len(case.k)), last)
    log("per-KV-head decode step")
    ca = write_cache(kvq, case, "fp8", "per_kv_head", ks, vs, rows=hist)
    cb = write_cache(kvq, case, "fp8", "per_kv_head", ks, vs, rows=hist)
    kvq.cache_write(ca, dev_bf16(case.k[last]), dev_bf16(case.v[last]),
                    dev(case.slots[last].astype(np.int64)))
    sc = kvq.Scales(1.0, 1.0, 1.0, 1.0)
    L = int(lens.max())
    a = kvq.decode_attention(ca, dev_bf16(case.q), dev(case.block_table),
                             dev(case.seq_lens), L, sc, out_dtype="f32")
    b = kvq.decode_step(cb, dev_bf16(case.q), dev_bf16(case.k[last]),
                        dev_bf16(case.v[last]), dev(case.block_table),
                        dev(case.seq_lens), L, sc, out_dtype="f32")
    assert np.array_equal(a.cpu().numpy(), b.cpu().numpy())
    pa, pb = read_pools(ca), read_pools(cb)
    for name in pa:
        assert np.array_equal(pa[name], pb[name]), name


@pytest.mark.parametrize("D,Hq,Hkv", [(256, 8, 4), (128, 16, 2)])
def test_prefill(kvq, D, Hq, Hkv):
    case = workloads.make_prefill_case(740 + D, [0, 300, 1000], [70, 129, 64], Hq, Hkv, D,
                                       table="perm")
    ks, vs = head_scales(D, Hkv), head_scales(D + 7, Hkv)
    log(f"per-KV-head prefill D={D}")
    c = write_cache(kvq, case, "fp8", "per_kv_head", ks, vs)
    got = run_prefill(kvq, c, case)
    want, bound = oracle_prefill(case, "per_kv_head", 1.0, ks, vs, p_bound=True)
    assert_close_with_p_rounding(got, want, bound, f"per-KV-head prefill D={D}")
