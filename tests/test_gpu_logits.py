"""GPU parity: paged query-key logits (kvq_paged_logits) against the float64 oracle.

Bar: entries past a row's visible length are -inf on both sides; visible entries
within 1e-6 of sum_d |q_d k_d| (the products are exact on the device, e4m3 and bf16
values being widened without rounding, and at most 256 of them are summed in float32:
the rounding of such a sum stays below 256 * 2^-24 of the sum of magnitudes).  The
magnitude sum is the oracle itself applied to |q| and |k|.
"""
import numpy as np
import pytest

import workloads
from oracle import cache as ocache, logits as ologits

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

from gpu_common import dev, dev_bf16, log, oracle_pools, write_cache  # noqa: E402

REL = 1e-6


@pytest.fixture(scope="module")
def kvq():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import fp8_quantized_paged_amd as k
    return k


def head_scales(case, seed=5):
    rng = np.random.default_rng(seed)
    return (rng.uniform(0.02, 0.2, case.num_kv_heads).astype(np.float32),
            rng.uniform(0.02, 0.2, case.num_kv_heads).astype(np.float32))


def run_case(kvq, case, dtype, mode, q_scale=1.0, k_scale=1.0, out_len=None):
    if out_len is None:
        out_len = -(-(int(case.seq_lens.max()) + 5) // 4) * 4
    if mode == "per_kv_head":
        ks, vs = head_scales(case)
    else:
        ks, vs = k_scale, k_scale
    c = write_cache(kvq, case, dtype, mode, ks, vs)
    sc = kvq.Scales(q_scale, k_scale if mode == "per_tensor" else 1.0, 1.0, 1.0)
    got = kvq.paged_logits(c, dev_bf16(case.q), dev(case.cu_rows), dev(case.row_lens),
                           dev(case.block_table), dev(case.seq_lens), out_len, sc)
    got = got.cpu().numpy().astype(np.float64)
    if dtype == "fp8":
        kp = ocache.dequantized(oracle_pools(case, mode, ks, vs), "k")
        _, qh = ocache.quantize_q(case.q, q_scale)
    else:  # bf16 cache: the raw rows
        kp = np.zeros((case.num_pages, case.num_kv_heads, 16, case.head_dim))
        kp[case.slots // 16, :, case.slots % 16] = case.k
        qh = case.q.astype(np.float64)
    want = ologits.paged_logits(qh, case.cu_rows, case.row_lens, kp, case.block_table,
                                out_len)
    mag = ologits.paged_logits(np.abs(qh), case.cu_rows, case.row_lens, np.abs(kp),
                               case.block_table, out_len)
    fin = np.isfinite(want)
    assert np.array_equal(np.isneginf(got), ~fin), "-inf pattern differs"
    err = np.abs(got[fin] - want[fin])
    bound = REL * mag[fin] + 1e-30
    bad = err > bound
    assert not bad.any(), (f"{bad.sum()} of {bad.size} logits off; worst "
                           f"{err.max():.3e} (bound {bound[np.argmax(err - bound)]:.3e})")
    return got


SHAPES = [(128, 4, 1), (64, 32, 8), (256, 16, 16), (128, 8, 2)]


@pytest.mark.parametrize("mode", ["per_token_head", "per_tensor", "per_kv_head"])
@pytest.mark.parametrize("D,Hq,Hkv", SHAPES)
def test_logits_fp8(kvq, mode, D, Hq, Hkv):
    # ragged: one token, page boundaries either side, several tiles; rows per request
    # 1..4 (the request's last tokens, causal prefixes)
    case = workloads.make_logits_case(500 + D + Hq, [1, 16, 17, 333, 700], [1, 4, 2, 3, 1],
                                      Hq, Hkv, D, table="perm")
    log(f"logits fp8 {mode} D={D} Hq={Hq} Hkv={Hkv}")
    run_case(kvq, case, "fp8", mode, k_scale=0.05 if mode == "per_tensor" else 1.0)


@pytest.mark.parametrize("D,Hq,Hkv", SHAPES)
def test_logits_bf16_cache(kvq, D, Hq, Hkv):
    case = workloads.make_logits_case(600 + D + Hq, [5, 64, 300], [2, 1, 3], Hq, Hkv, D,
                                      table="perm")
    log(f"logits bf16 D={D} Hq={Hq} Hkv={Hkv}")
    run_case(kvq, case, "bf16", "per_token_head")


def test_logits_q_scale_and_many_rows(kvq):
    """q_scale != 1 and a request with more than 32 (row, head) pairs per key head
    (several column chunks), rows that see the whole cache."""
    case = workloads.make_logits_case(701, [40, 1000], [20, 9], 8, 2, 128, table="perm",
                                      causal_rows=False)
    log("logits q_scale 0.5, 29 rows")
    run_case(kvq, case, "fp8", "per_token_head", q_scale=0.5)


def test_logits_chunk_sets(kvq):
    """Requests averaging more than 32 (row, head) pairs per key head: the launch also
    splits over 32-pair chunks (7 chunk sets here), a request with more chunks loops over
    them (600 pairs), one has a single chunk and one none; stores through the lane-quad
    transpose.  FP8 with per-token-head scales and a bf16 cache."""
    case = workloads.make_logits_case(741, [900, 40, 17, 300], [150, 3, 0, 61], 8, 2, 128,
                                      table="perm")
    log("logits chunk sets fp8, 214 rows")
    run_case(kvq, case, "fp8", "per_token_head", q_scale=0.25)
    case = workloads.make_logits_case(742, [130, 517], [100, 37], 4, 1, 64, table="perm")
    log("logits chunk sets bf16, 137 rows")
    run_case(kvq, case, "bf16", "per_token_head")


@pytest.mark.parametrize("Hq,Hkv,rows,mode", [
    (6, 2, [50, 7], "per_tensor"),        # group 3: lane-quad transposed stores
    (32, 2, [5, 3], "per_kv_head"),       # group 16: swapped operands, 5 chunks per row
    (64, 1, [1, 2, 1], "per_token_head"), # group 64: a chunk is 32 heads of one row
])
def test_logits_store_forms(kvq, Hq, Hkv, rows, mode):
    """Every store form the launch picks for requests of more than 8 pairs: a group
    size that is not a power of two, and power-of-two groups below and above 32."""
    case = workloads.make_logits_case(750 + Hq, [300, 45, 1000][:len(rows)], rows, Hq, Hkv,
                                      128, table="perm")
    log(f"logits store forms Hq={Hq} Hkv={Hkv} rows={rows} {mode}")
    run_case(kvq, case, "fp8", mode, k_scale=0.05 if mode == "per_tensor" else 1.0)


def test_logits_edges(kvq):
    """Empty requests, rows with no visible key, and an output narrower than the cache
    (keys past out_len are not written) or wider (all -inf past the visible keys)."""
    case = workloads.make_logits_case(711, [0, 3, 260, 16], [2, 3, 1, 0], 4, 1, 64,
                                      table="perm")
    log("logits edges")
    run_case(kvq, case, "fp8", "per_token_head", out_len=128)
    run_case(kvq, case, "fp8", "per_token_head", out_len=512)


def test_logits_wide_output_and_empty_cache(kvq):
    """Output rows so long (8,200,000 entries, one query head per key head) that a
    32-pair column chunk spans more than 2 GB of output: the kernel then stores without
    the buffer resource; the first 512 entries of every row against the oracle, the
    rest -inf.  And a cache with no pages at all: every logit -inf."""
    case = workloads.make_logits_case(731, [300, 40], [2, 1], 2, 2, 64, table="perm")
    out_len, head = 8_200_000, 512
    c = write_cache(kvq, case, "fp8", "per_token_head")
    log("logits wide output rows (plain stores)")
    got = kvq.paged_logits(c, dev_bf16(case.q), dev(case.cu_rows), dev(case.row_lens),
                           dev(case.block_table), dev(case.seq_lens), out_len,
                           kvq.Scales(1.0, 1.0, 1.0, 1.0))
    tail_inf = bool(torch.isneginf(got[:, :, head:]).all())
    got = got[:, :, :head].cpu().numpy().astype(np.float64)
    assert tail_inf, "entries past the visible keys must be -inf"
    kp = ocache.dequantized(oracle_pools(case, "per_token_head", 1.0, 1.0), "k")
    _, qh = ocache.quantize_q(case.q, 1.0)
    want = ologits.paged_logits(qh, case.cu_rows, case.row_lens, kp, case.block_table, head)
    mag = ologits.paged_logits(np.abs(qh), case.cu_rows, case.row_lens, np.abs(kp),
                               case.block_table, head)
    fin = np.isfinite(want)
    assert np.array_equal(np.isneginf(got), ~fin), "-inf pattern differs"
    assert (np.abs(got[fin] - want[fin]) <= REL * mag[fin] + 1e-30).all()

    log("logits empty cache")
    c0 = kvq.PagedCache(0, 2, 64, "fp8", "per_token_head")
    q = dev_bf16(case.q)
    cu = dev(np.array([0, 1, 3], dtype=np.int32))
    zeros = dev(np.zeros(3, dtype=np.int32))
    bt = dev(np.zeros((2, 1), dtype=np.int32))
    got0 = kvq.paged_logits(c0, q, cu, zeros, bt, zeros[:2], 64, kvq.Scales(1.0, 1.0, 1.0, 1.0))
    assert bool(torch.isneginf(got0).all())


def test_logits_sampled_at_full_size(kvq):
    """The bench's workload (32 requests x 20,000 cached tokens, 4 query heads on one
    key head, D 128, one query row each), every logit of 4 sampled requests checked."""
    B, L = 32, 20000
    case = workloads.make_logits_case(721, [L] * B, [1] * B, 4, 1, 128, table="perm")
    out_len = L
    c = write_cache(kvq, case, "fp8", "per_token_head")
    got = kvq.paged_logits(c, dev_bf16(case.q), dev(case.cu_rows), dev(case.row_lens),
                           dev(case.block_table), dev(case.seq_lens), out_len,
                           kvq.Scales(1.0, 1.0, 1.0, 1.0)).cpu().numpy().astype(np.float64)
    _, qh = ocache.quantize_q(case.q, 1.0)
    for b in (0, 7, 19, 31):
        sel = np.nonzero(case.token_seq == b)[0]
        pools = ocache.new_pools(case.num_pages, 1, 128)
        ocache.cache_write(pools, case.k[sel], case.v[sel], case.slots[sel], "per_token_head")
        kp = ocache.dequantized(pools, "k")
        cu = np.array([0, 1])
        want = ologits.paged_logits(qh[b:b + 1], cu, case.row_lens[b:b + 1], kp,
                                    case.block_table[b:b + 1], out_len)
        mag = ologits.paged_logits(np.abs(qh[b:b + 1]), cu, case.row_lens[b:b + 1],
                                   np.abs(kp), case.block_table[b:b + 1], out_len)
        err = np.abs(got[b:b + 1] - want)
        assert (err <= REL * mag + 1e-30).all(), f"request {b}: worst {err.max():.3e}"
    log("logits full size sampled")


def test_logits_many_rows_sampled_at_full_size(kvq):
    """The bench's many-rows workload (one request of 8,192 causal query rows over its
    8,192 cached tokens, 4 query heads on one key head, D 128; 1 GiB of logits, the
    swapped-operand store form over 6,144 workgroups): every logit of 10 sampled rows,
    chosen across chunk boundaries (8 rows per 32-pair chunk) and the request's ends."""
    R = L = 8192
    case = workloads.make_logits_case(761, [L], [R], 4, 1, 128, table="perm")
    c = write_cache(kvq, case, "fp8", "per_token_head")
    out = kvq.paged_logits(c, dev_bf16(case.q), dev(case.cu_rows), dev(case.row_lens),
                           dev(case.block_table), dev(case.seq_lens), L,
                           kvq.Scales(1.0, 1.0, 1.0, 1.0))
    rows = np.array([0, 1, 7, 8, 255, 256, 4095, 4100, 8190, 8191])
    got = out[torch.from_numpy(rows).to(out.device)].cpu().numpy().astype(np.float64)
    del out
    _, qh = ocache.quantize_q(case.q[rows], 1.0)
    pools = ocache.new_pools(case.num_pages, 1, 128)
    ocache.cache_write(pools, case.k, case.v, case.slots, "per_token_head")
    kp = ocache.dequantized(pools, "k")
    cu = np.array([0, len(rows)])
    want = ologits.paged_logits(qh, cu, case.row_lens[rows], kp, case.block_table, L)
    mag = ologits.paged_logits(np.abs(qh), cu, case.row_lens[rows], np.abs(kp),
                               case.block_table, L)
    fin = np.isfinite(want)
    assert np.array_equal(np.isneginf(got), ~fin), "-inf pattern differs"
    err = np.abs(got[fin] - want[fin])
    assert (err <= REL * mag[fin] + 1e-30).all(), f"worst {err.max():.3e}"
    log("logits many rows full size sampled")
