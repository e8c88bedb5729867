"""GPU: decode steps captured in a HIP graph (torch.cuda.CUDAGraph) replay to the same
bits as the eager calls.

A serving loop replays one captured step per token; the library launches on torch's
current stream, allocates nothing and resets its own split counters, so the capture
holds only its kernels.  Each replay is checked against the eager result, with eager
work and a synchronisation between replays.
"""
import numpy as np
import pytest

import workloads

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

from gpu_common import dev, dev_bf16, log, read_pools, write_cache  # noqa: E402


@pytest.fixture(scope="module")
def kvq():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import fp8_quantized_paged_amd as k
    return k


# (dtype, mode, D, Hq, Hkv, window): vector form, both matrix-core forms, bf16 skip path
LAYERS = [("fp8", "per_token_head", 128, 32, 8, 0), ("fp8", "per_tensor", 64, 64, 8, 0),
          ("fp8", "per_token_head", 128, 64, 8, 0), ("bf16", "per_token_head", 64, 64, 8, 128)]


def make_layer(kvq, i, dtype, mode, D, Hq, Hkv, window):
    case = workloads.make_decode_case(600 + i, [300, 17, 1, 1200], Hq, Hkv, D, table="perm",
                                      window=window)
    starts = np.concatenate([[0], np.cumsum(case.seq_lens)[:-1]])
    last = starts + case.seq_lens - 1
    hist = np.setdiff1d(np.arange(len(case.k)), last)
    c = write_cache(kvq, case, dtype, mode, rows=hist)
    B = len(case.seq_lens)
    ws = kvq.decode_workspace(c, B, Hq, int(case.seq_lens.max()), window, 0,
                              torch.device("cuda"))
    return dict(c=c, q=dev_bf16(case.q), kn=dev_bf16(case.k[last]), vn=dev_bf16(case.v[last]),
                bt=dev(case.block_table), sl=dev(case.seq_lens), L=int(case.seq_lens.max()),
                window=window, ws=ws, out=torch.empty((B, Hq, D), dtype=torch.float32,
                                                      device="cuda"))


def step(kvq, layers):
    for ly in layers:
        kvq.decode_step(ly["c"], ly["q"], ly["kn"], ly["vn"], ly["bt"], ly["sl"], ly["L"],
                        window=ly["window"], out=ly["out"], out_dtype="f32",
                        workspace=ly["ws"])


def test_graph_replays_match_eager(kvq):
    log("graph capture of decode steps")
    eager = [make_layer(kvq, i, *spec) for i, spec in enumerate(LAYERS)]
    step(kvq, eager)
    torch.cuda.synchronize()
    want = [ly["out"].cpu().numpy() for ly in eager]
    want_pools = [read_pools(ly["c"]) for ly in eager]

    layers = [make_layer(kvq, i, *spec) for i, spec in enumerate(LAYERS)]
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step(kvq, layers)  # warm-up on a side stream, as capture requires
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step(kvq, layers)
    torch.cuda.synchronize()
    for rep in range(4):
        for ly in layers:
            ly["out"].fill_(float("nan"))
        g.replay()
        torch.cuda.synchronize()
        for i, ly in enumerate(layers):
            got = ly["out"].cpu().numpy()
            assert np.array_equal(got, want[i]), f"replay {rep} layer {i}"
        # eager work between the replays
        x = torch.randn(1 << 20, device="cuda")
        float(x.sum())
        torch.cuda.synchronize()
    for i, ly in enumerate(layers):
        pools = read_pools(ly["c"])
        for name in pools:
            assert np.array_equal(pools[name], want_pools[i][name]), f"layer {i} {name}"
