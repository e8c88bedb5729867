"""GPU: kvq_decode_attention_noalloc (the library's own device scratch instead of a
workspace) gives the same outputs as kvq_decode_attention on the same inputs, bit for
bit (same kernels, same split plan), on consecutive calls whose shapes shrink, and
refuses arguments whose partials exceed its scratch."""
import numpy as np
import pytest

import workloads

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

from gpu_common import (assert_close_to_oracle, dev, dev_bf16, log,  # noqa: E402
                        oracle_pools, write_cache)
from oracle import attention, cache as ocache  # noqa: E402


@pytest.fixture(scope="module")
def kvq():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import fp8_quantized_paged_amd as k
    return k


def _oracle(case):
    pools = oracle_pools(case, "per_token_head")
    _, qh = ocache.quantize_q(case.q, 1.0)
    return attention.decode(qh, ocache.dequantized(pools, "k"), ocache.dequantized(pools, "v"),
                            case.block_table, case.seq_lens)


def test_noalloc_matches_workspace_entry_point(kvq):
    sc = kvq.Scales(1.0, 1.0, 1.0, 1.0)
    big = workloads.make_decode_case(81, [5000, 3000, 4100, 17, 2600, 0, 999, 4500], 32, 8,
                                     128, table="perm", outliers=4)
    small = workloads.make_decode_case(82, [1800, 40], 32, 8, 128, table="perm")
    for case, name in ((big, "8 sequences"), (small, "2 sequences, shorter")):
        log(f"noalloc decode: {name}")
        c = write_cache(kvq, case, "fp8", "per_token_head")
        L = int(case.seq_lens.max())
        q, bt, sl = dev_bf16(case.q), dev(case.block_table), dev(case.seq_lens)
        for pps in (4, 0):
            assert kvq.decode_workspace_bytes(c, len(case.seq_lens), 32, L, 0, pps) > 0
            ref = kvq.decode_attention(c, q, bt, sl, L, sc, pages_per_split=pps,
                                       out_dtype="f32")
            out = torch.empty_like(ref)
            got = kvq.decode_attention_noalloc(c, q, bt, sl, L, sc, pages_per_split=pps,
                                               out=out, out_dtype="f32")
            torch.cuda.synchronize()
            assert got.data_ptr() == out.data_ptr()
            assert torch.equal(got, ref), (name, pps)
            assert_close_to_oracle(got.cpu().numpy(), _oracle(case), f"noalloc {name}")


def test_noalloc_refuses_oversized_partials(kvq):
    # 64 sequences x 32 q heads x 256 splits x 130 floats = 272 MB of partials
    c = kvq.PagedCache(16, 8, 128, "fp8", "per_token_head")
    q = torch.zeros((64, 32, 128), dtype=torch.bfloat16, device="cuda")
    bt = torch.zeros((64, 256), dtype=torch.int32, device="cuda")
    sl = torch.zeros(64, dtype=torch.int32, device="cuda")
    assert kvq.decode_workspace_bytes(c, 64, 32, 4096, 0, 1) > kvq.DECODE_SCRATCH_BYTES
    with pytest.raises(kvq.KvqError) as e:
        kvq.decode_attention_noalloc(c, q, bt, sl, 4096, pages_per_split=1)
    assert e.value.status == kvq.binding.ERR_WORKSPACE
