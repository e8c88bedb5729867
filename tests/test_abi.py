"""CPU tests of the C ABI: the library loads, exports every declared symbol, and its
host-only logic (scale resolution, skip policy, argument checks) behaves as stated.
No device work is enqueued by any call here."""
import ctypes

import numpy as np
import pytest

from oracle import scales as oscales

import fp8_quantized_paged_amd as kvq  # noqa: E402  (a missing or stale library fails here)

from test_oracle_cache import read_scale_cases  # noqa: E402


def test_exports_every_declared_function():
    names = kvq.header_functions()
    assert len(names) >= 10
    missing = [n for n in names if not kvq.exported(n)]
    assert not missing, missing


def test_abi_version():
    assert kvq.abi_version() == 1


@pytest.mark.parametrize("case", list(read_scale_cases()))
def test_resolve_scales_matches_oracle(case):
    mode, raw, rhs = case
    if rhs == ["error"]:
        with pytest.raises(kvq.KvqError):
            kvq.resolve_scales(mode, *raw)
        with pytest.raises(oscales.ScaleError):
            oscales.resolve(mode, *raw)
        return
    got, warn = kvq.resolve_scales(mode, *raw)
    want, wwarn = oscales.resolve(mode, *raw)
    assert got.as_tuple() == (want.q_scale, want.k_scale, want.v_scale, want.prob_scale)
    assert warn == wwarn


def test_resolve_scales_random_against_oracle():
    rng = np.random.default_rng(0)
    vals = [-1.0, 0.0, 0.25, 1.0, 3.5, -2.0]
    for _ in range(300):
        raw = [float(rng.choice(vals)) for _ in range(4)]
        for mode in ("per_tensor", "per_token_head"):
            try:
                want, wwarn = oscales.resolve(mode, *raw)
            except oscales.ScaleError:
                with pytest.raises(kvq.KvqError):
                    kvq.resolve_scales(mode, *raw)
                continue
            got, warn = kvq.resolve_scales(mode, *raw)
            assert got.as_tuple() == (want.q_scale, want.k_scale, want.v_scale,
                                      want.prob_scale)
            assert warn == wwarn


@pytest.mark.parametrize("window", [0, 1, 128])
@pytest.mark.parametrize("flags", [0, 1])
def test_layer_kv_dtype_matches_oracle(window, flags):
    assert kvq.layer_kv_dtype(window, flags) == oscales.layer_kv_dtype(window, flags)


def _desc(**kw):
    d = dict(dtype=kvq.FP8_E4M3, mode=kvq.PER_TOKEN_HEAD, num_pages=4, page_size=16,
             num_kv_heads=2, head_dim=128, k_pages=4096, v_pages=8192, k_scales=256,
             v_scales=512)
    d.update(kw)
    return kvq.CacheDesc(**d)


def _lib():
    return kvq.binding._lib


@pytest.mark.parametrize("bad,status", [
    (dict(head_dim=96), kvq.binding.ERR_UNSUPPORTED),
    (dict(page_size=32), kvq.binding.ERR_UNSUPPORTED),
    (dict(num_kv_heads=0), kvq.binding.ERR_INVALID_ARG),
    (dict(k_pages=None), kvq.binding.ERR_INVALID_ARG),
    (dict(k_pages=4100), kvq.binding.ERR_INVALID_ARG),
    (dict(k_scales=None), kvq.binding.ERR_INVALID_ARG),
    (dict(dtype=7), kvq.binding.ERR_UNSUPPORTED),
])
def test_cache_descriptor_checks(bad, status):
    d = _desc(**bad)
    st = _lib().kvq_cache_write(ctypes.byref(d), 16, 32, 0, 64, 1, 1.0, 1.0, None)
    assert st == status, kvq.last_error()
    assert kvq.last_error()


def test_cache_write_argument_checks():
    d = _desc()
    L = _lib()
    assert L.kvq_cache_write(None, 16, 32, 0, 64, 1, 1.0, 1.0, None) == kvq.binding.ERR_INVALID_ARG
    assert L.kvq_cache_write(ctypes.byref(d), 16, 32, 0, 64, -1, 1.0, 1.0, None) == kvq.binding.ERR_INVALID_ARG
    assert L.kvq_cache_write(ctypes.byref(d), 16, 32, 0, 64, 0, 1.0, 1.0, None) == kvq.binding.OK
    assert L.kvq_cache_write(ctypes.byref(d), None, 32, 0, 64, 1, 1.0, 1.0, None) == kvq.binding.ERR_INVALID_ARG
    assert L.kvq_cache_write(ctypes.byref(d), 16, 32, 100, 64, 1, 1.0, 1.0, None) == kvq.binding.ERR_INVALID_ARG
    assert L.kvq_cache_write(ctypes.byref(d), 8, 32, 0, 64, 1, 1.0, 1.0, None) == kvq.binding.ERR_INVALID_ARG
    pt = _desc(mode=kvq.PER_TENSOR)
    assert L.kvq_cache_write(ctypes.byref(pt), 16, 32, 0, 64, 1, 0.0, 1.0, None) == kvq.binding.ERR_INVALID_ARG
    assert L.kvq_cache_write(ctypes.byref(pt), 16, 32, 0, 64, 1, -1.0, 1.0, None) == kvq.binding.ERR_INVALID_ARG


def test_per_kv_head_mode():
    """Per-KV-head caches need their scale arrays; resolution follows the per-tensor
    rules for one head's (k, v) pair."""
    L = _lib()
    d = _desc(mode=kvq.PER_KV_HEAD, k_scales=None, v_scales=None)
    assert L.kvq_cache_write(ctypes.byref(d), 16, 32, 0, 64, 1, 1.0, 1.0, None) == kvq.binding.ERR_INVALID_ARG
    d = _desc(mode=kvq.PER_KV_HEAD, k_scales=258, v_scales=512)     # misaligned array
    assert L.kvq_cache_write(ctypes.byref(d), 16, 32, 0, 64, 1, 1.0, 1.0, None) == kvq.binding.ERR_INVALID_ARG
    d = _desc(mode=kvq.PER_KV_HEAD)
    assert L.kvq_cache_write(ctypes.byref(d), 16, 32, 0, 64, 0, 1.0, 1.0, None) == kvq.binding.OK
    # the call's per-tensor scalars are not used in this mode: 0 is no error here
    assert L.kvq_cache_write(ctypes.byref(d), 16, 32, 0, 64, 0, 0.0, 0.0, None) == kvq.binding.OK
    for raw in [(-1.0, -1.0, -1.0, -1.0), (0.5, 0.25, 2.0, 0.125), (0.3, -1.0, -1.0, 4.0)]:
        got, warn = kvq.resolve_scales("per_kv_head", *raw)
        want, wwarn = oscales.resolve("per_kv_head", *raw)
        # the library holds float32 values
        assert got.as_tuple() == tuple(float(np.float32(x)) for x in (
            want.q_scale, want.k_scale, want.v_scale, want.prob_scale))
        assert warn == wwarn
        assert got.as_tuple() == kvq.resolve_scales("per_tensor", *raw)[0].as_tuple()


def test_decode_workspace_and_checks():
    d = _desc()
    L = _lib()
    n = ctypes.c_size_t()
    assert L.kvq_decode_workspace_bytes(ctypes.byref(d), 8, 32, 20000, 0, 0, ctypes.byref(n)) == 0
    C = kvq.DECODE_COUNTER_BYTES   # fixed counter prefix, whatever the shape
    assert n.value > C
    assert (n.value - C) % (8 * 32 * (128 + 2) * 4) == 0
    # explicit pages_per_split: splits = ceil(1250 / 10) = 125
    assert L.kvq_decode_workspace_bytes(ctypes.byref(d), 8, 32, 20000, 0, 10, ctypes.byref(n)) == 0
    assert n.value == C + 8 * 32 * 125 * 130 * 4
    # one long sequence: the automatic split count stops at 32 per (sequence, KV head)
    # (8,192 pages -> 256 pages per split)
    one = _desc(mode=kvq.PER_TENSOR)
    assert L.kvq_decode_workspace_bytes(ctypes.byref(one), 1, 32, 131072, 0, 0, ctypes.byref(n)) == 0
    assert n.value == C + 1 * 32 * 32 * 130 * 4
    # a window bounds the visible pages: 128 keys span at most 9 pages
    assert L.kvq_decode_workspace_bytes(ctypes.byref(d), 8, 32, 20000, 128, 4, ctypes.byref(n)) == 0
    assert n.value == C + 8 * 32 * 3 * 130 * 4
    # more than KVQ_DECODE_MAX_SPLIT_UNITS (sequence, KV head) pairs only without splits
    # (this descriptor has 2 KV heads: 32,769 sequences are 65,538 pairs)
    assert L.kvq_decode_workspace_bytes(ctypes.byref(d), 32769, 32, 20000, 0, 0,
                                        ctypes.byref(n)) == kvq.binding.ERR_UNSUPPORTED
    assert L.kvq_decode_workspace_bytes(ctypes.byref(d), 32769, 32, 4096, 0, 0,
                                        ctypes.byref(n)) == 0 and n.value == 0
    assert L.kvq_decode_workspace_bytes(ctypes.byref(d), 32768, 32, 20000, 0, 0,
                                        ctypes.byref(n)) == 0 and n.value > C
    assert L.kvq_decode_workspace_bytes(ctypes.byref(d), 8, 24, 20000, 0, 0, ctypes.byref(n)) == kvq.binding.ERR_UNSUPPORTED
    assert L.kvq_decode_workspace_bytes(ctypes.byref(d), 8, 33, 20000, 0, 0, ctypes.byref(n)) == kvq.binding.ERR_INVALID_ARG
    assert L.kvq_decode_workspace_bytes(ctypes.byref(d), 8, 32, 20000, 0, 257, ctypes.byref(n)) == kvq.binding.ERR_INVALID_ARG
    sc = kvq.Scales(1.0, 1.0, 1.0, 1.0)
    args = lambda ws, wsb, outdt=kvq.BF16, q=4096, scales=ctypes.byref(sc): (
        ctypes.byref(d), q, 8, 32, 4096, 1250, 4096, 20000, scales, 0, 0.0, 10, 4096,
        outdt, ws, wsb, None)
    need = C + 8 * 32 * 125 * 130 * 4
    assert L.kvq_decode_attention(*args(None, 0)) == kvq.binding.ERR_WORKSPACE
    assert L.kvq_decode_attention(*args(4096, need - 1)) == kvq.binding.ERR_WORKSPACE
    assert L.kvq_decode_attention(*args(4096, need, outdt=kvq.FP8_E4M3)) == kvq.binding.ERR_UNSUPPORTED
    assert L.kvq_decode_attention(*args(4096, need, q=4100)) == kvq.binding.ERR_INVALID_ARG
    assert L.kvq_decode_attention(*args(4096, need, scales=None)) == kvq.binding.ERR_INVALID_ARG
    bad = kvq.Scales(0.0, 1.0, 1.0, 1.0)
    assert L.kvq_decode_attention(*args(4096, need, scales=ctypes.byref(bad))) == kvq.binding.ERR_INVALID_ARG

    # decode step: the same checks, plus the new-token rows (non-null, 16-byte aligned);
    # every call below fails before anything is enqueued
    step = lambda kn, vn, ws, wsb, outdt=kvq.BF16: (
        ctypes.byref(d), 4096, kn, vn, 8, 32, 4096, 1250, 4096, 20000, ctypes.byref(sc), 0,
        0.0, 10, 4096, outdt, ws, wsb, None)
    assert L.kvq_decode_step(*step(None, 8192, 4096, need)) == kvq.binding.ERR_INVALID_ARG
    assert L.kvq_decode_step(*step(8192, None, 4096, need)) == kvq.binding.ERR_INVALID_ARG
    assert L.kvq_decode_step(*step(8200, 8192, 4096, need)) == kvq.binding.ERR_INVALID_ARG
    assert L.kvq_decode_step(*step(8192, 8192, None, 0)) == kvq.binding.ERR_WORKSPACE
    assert L.kvq_decode_step(*step(8192, 8192, 4096, need, kvq.FP8_E4M3)) == kvq.binding.ERR_UNSUPPORTED


def test_quantize_argument_checks():
    L = _lib()
    assert L.kvq_quantize_fp8(16, -1, 1.0, 16, None) == kvq.binding.ERR_INVALID_ARG
    assert L.kvq_quantize_fp8(16, 0, 1.0, 16, None) == kvq.binding.OK
    assert L.kvq_quantize_fp8(None, 8, 1.0, 16, None) == kvq.binding.ERR_INVALID_ARG
    assert L.kvq_quantize_fp8(17, 8, 1.0, 16, None) == kvq.binding.ERR_INVALID_ARG


def test_status_strings():
    for s in range(5):
        assert kvq.status_string(s)


def test_single_hip_runtime_in_process():
    """libkvq must share torch's HIP runtime: exactly one libamdhip64 is mapped even
    though this package may be imported before torch."""
    import subprocess
    import sys
    code = ("import fp8_quantized_paged_amd, torch\n"
            "libs = {l.split()[-1] for l in open('/proc/self/maps') if 'libamdhip64' in l}\n"
            "print(len(libs))\n")
    out = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True,
                         cwd=__import__("os").path.dirname(__import__("os").path.dirname(
                             __import__("os").path.abspath(__file__))))
    assert out.returncode == 0, out.stderr
    assert out.stdout.strip() == "1"


def test_mfma_probe_library_loads_and_checks_arguments():
    """The measurement probe beside the library (bench.py only) is built with it, loads
    without a GPU, and refuses bad arguments before launching anything."""
    import os
    path = os.path.join(os.path.dirname(kvq.__file__), "libkvq_probe.so")
    assert os.path.exists(path), "build() also builds libkvq_probe.so"
    lib = ctypes.CDLL(path)
    fn = lib.kvq_probe_mfma_rate
    fn.restype = ctypes.c_int
    fn.argtypes = [ctypes.c_int32, ctypes.c_int32, ctypes.c_void_p, ctypes.c_void_p]
    assert fn(0, 10, None, None) == 1
    assert fn(256, 0, None, None) == 1
    assert fn(256, 10, None, None) == 1   # no output buffer
