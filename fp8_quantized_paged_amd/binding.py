"""ctypes binding of libkvq.so.  Argument marshalling only: every step of the
computation runs in the library's HIP kernels; torch provides device memory and the
stream.  Names follow the C ABI in include/kvq.h (without the ``kvq_`` prefix).

There is no fallback: if libkvq.so is missing or fails to load, importing this
module raises ImportError.
"""
from __future__ import annotations

import ctypes
import os
import re

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libkvq.so")
HEADER = os.path.join(os.path.dirname(HERE), "include", "kvq.h")

if not os.path.exists(LIB_PATH):
    raise ImportError(f"{LIB_PATH} is not built; run python -m fp8_quantized_paged_amd.build")

# torch ships its own HIP runtime.  Device pointers and streams handed to libkvq come
# from torch, so libkvq must bind to that same runtime: import torch first, so that
# the loader resolves libkvq's libamdhip64 dependency to the copy already loaded.
import torch as _torch_mod  # noqa: E402,F401

try:
    _lib = ctypes.CDLL(LIB_PATH)
except OSError as e:  # pragma: no cover - depends on the machine
    raise ImportError(f"cannot load {LIB_PATH}: {e}") from e


def _stale_check() -> None:
    """Refuse a library built from other sources than the tree's (a stale build)."""
    from .build import source_hash
    try:
        built = ctypes.string_at(ctypes.addressof(
            ctypes.c_char.in_dll(_lib, "kvq_build_source_hash"))).decode()
    except ValueError:
        built = "(no source hash recorded)"
    want = source_hash()
    if built != want:
        raise ImportError(f"{LIB_PATH} is stale: built from sources {built}, the tree is "
                          f"{want}; rebuild with python -m fp8_quantized_paged_amd.build")


_stale_check()


def _hip_runtimes_mapped() -> set:
    libs = set()
    with open("/proc/self/maps") as f:
        for line in f:
            path = line.split()[-1]
            if "libamdhip64" in path:
                libs.add(os.path.realpath(path))
    return libs


if len(_hip_runtimes_mapped()) > 1:
    raise ImportError("two HIP runtimes are loaded in this process "
                      f"({sorted(_hip_runtimes_mapped())}); import torch before any other "
                      "HIP library so libkvq shares torch's runtime")

# ---- enums and structs (mirror include/kvq.h) -------------------------------------
OK, ERR_INVALID_ARG, ERR_UNSUPPORTED, ERR_WORKSPACE, ERR_HIP = range(5)
BF16, FP8_E4M3, F32 = 0, 1, 2
PER_TENSOR, PER_TOKEN_HEAD, PER_KV_HEAD = 0, 1, 2
WARN_UNCALIBRATED_Q_OR_PROB = 1
SKIP_SLIDING_WINDOW = 1
PAGE_SIZE = 16
# fixed counter prefix of every decode workspace (include/kvq.h)
DECODE_MAX_SPLIT_UNITS = 65536
DECODE_COUNTER_BYTES = 4 * DECODE_MAX_SPLIT_UNITS
DECODE_SCRATCH_BYTES = 32 * 1024 * 1024
_MODES = {"per_tensor": PER_TENSOR, "per_token_head": PER_TOKEN_HEAD,
          "per_kv_head": PER_KV_HEAD}
_DTYPES = {"bf16": BF16, "fp8": FP8_E4M3, "f32": F32}
ACCUM_MFMA_CHAIN, ACCUM_VALU_ADD = 0, 1
ACCUMULATIONS = {"mfma_chain": ACCUM_MFMA_CHAIN, "valu_add": ACCUM_VALU_ADD}


class Scales(ctypes.Structure):
    _fields_ = [("q_scale", ctypes.c_float), ("k_scale", ctypes.c_float),
                ("v_scale", ctypes.c_float), ("prob_scale", ctypes.c_float)]

    def as_tuple(self):
        return (self.q_scale, self.k_scale, self.v_scale, self.prob_scale)


class CacheDesc(ctypes.Structure):
    _fields_ = [("dtype", ctypes.c_int), ("mode", ctypes.c_int),
                ("num_pages", ctypes.c_int32), ("page_size", ctypes.c_int32),
                ("num_kv_heads", ctypes.c_int32), ("head_dim", ctypes.c_int32),
                ("k_pages", ctypes.c_void_p), ("v_pages", ctypes.c_void_p),
                ("k_scales", ctypes.c_void_p), ("v_scales", ctypes.c_void_p)]


class KvqError(RuntimeError):
    def __init__(self, status: int, where: str):
        msg = _lib.kvq_last_error().decode()
        super().__init__(f"{where}: {_lib.kvq_status_string(status).decode()} ({msg})")
        self.status = status


_i32, _i64, _f32, _p, _sz = (ctypes.c_int32, ctypes.c_int64, ctypes.c_float,
                             ctypes.c_void_p, ctypes.c_size_t)
_PD = ctypes.POINTER(CacheDesc)
_SIGS = {
    "kvq_abi_version": (_i32, []),
    "kvq_status_string": (ctypes.c_char_p, [ctypes.c_int]),
    "kvq_last_error": (ctypes.c_char_p, []),
    "kvq_resolve_scales": (ctypes.c_int, [ctypes.c_int, _f32, _f32, _f32, _f32,
                                          ctypes.POINTER(Scales),
                                          ctypes.POINTER(ctypes.c_uint32)]),
    "kvq_layer_kv_dtype": (ctypes.c_int, [_i32, ctypes.c_uint32]),
    "kvq_cache_write": (ctypes.c_int, [_PD, _p, _p, _i64, _p, _i32, _f32, _f32, _p]),
    "kvq_quantize_fp8": (ctypes.c_int, [_p, _i64, _f32, _p, _p]),
    "kvq_decode_workspace_bytes": (ctypes.c_int, [_PD, _i32, _i32, _i32, _i32, _i32,
                                                  ctypes.POINTER(_sz)]),
    "kvq_decode_attention": (ctypes.c_int, [_PD, _p, _i32, _i32, _p, _i32, _p, _i32,
                                            ctypes.POINTER(Scales), _i32, _f32, _i32,
                                            _p, ctypes.c_int, _p, _sz, _p]),
    "kvq_decode_attention_noalloc": (ctypes.c_int, [_PD, _p, _i32, _i32, _p, _i32, _p, _i32,
                                                    ctypes.POINTER(Scales), _i32, _f32, _i32,
                                                    _p, ctypes.c_int, _p]),
    "kvq_decode_step": (ctypes.c_int, [_PD, _p, _p, _p, _i32, _i32, _p, _i32, _p, _i32,
                                       ctypes.POINTER(Scales), _i32, _f32, _i32,
                                       _p, ctypes.c_int, _p, _sz, _p]),
    "kvq_prefill_attention": (ctypes.c_int, [_PD, _p, _p, _i32, _i32, _p, _i32, _p,
                                             _i32, ctypes.POINTER(Scales), _i32, _i32,
                                             _f32, _p, ctypes.c_int, _p]),
    "kvq_prefill_attention_accum": (ctypes.c_int, [_PD, _p, _p, _i32, _i32, _p, _i32, _p,
                                                   _i32, ctypes.POINTER(Scales), _i32, _i32,
                                                   _f32, _p, ctypes.c_int, ctypes.c_int, _p]),
    "kvq_prefill_workspace_bytes": (ctypes.c_size_t, [_PD, _i32, _i32, _i32]),
    "kvq_prefill_attention_ws": (ctypes.c_int, [_PD, _p, _p, _i32, _i32, _p, _i32, _p, _i32,
                                                ctypes.POINTER(Scales), _i32, _i32, _f32, _p,
                                                ctypes.c_int, _p, ctypes.c_size_t, _p]),
    "kvq_paged_logits": (ctypes.c_int, [_PD, _p, _p, _i32, _i32, _i32, _p, _p, _i32, _p,
                                        ctypes.POINTER(Scales), _p, _i32, _p]),
}
for _name, (_res, _args) in _SIGS.items():
    if hasattr(_lib, _name):
        _fn = getattr(_lib, _name)
        _fn.restype = _res
        _fn.argtypes = _args


def header_functions() -> list[str]:
    """Names of the functions include/kvq.h declares."""
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(kvq_[a-z0-9_]+)\s*\(", text)))


def exported(name: str) -> bool:
    return hasattr(_lib, name)


def _check(status: int, where: str) -> None:
    if status != OK:
        raise KvqError(status, where)


# ---- host-only helpers ---------------------------------------------------------------

def abi_version() -> int:
    return _lib.kvq_abi_version()


def status_string(s: int) -> str:
    return _lib.kvq_status_string(s).decode()


def last_error() -> str:
    return _lib.kvq_last_error().decode()


def resolve_scales(mode: str, k: float, v: float, q: float, prob: float):
    out = Scales()
    warn = ctypes.c_uint32(0)
    _check(_lib.kvq_resolve_scales(_MODES[mode], k, v, q, prob, ctypes.byref(out),
                                   ctypes.byref(warn)), "resolve_scales")
    return out, warn.value


def layer_kv_dtype(window: int, skip_flags: int) -> str:
    return {BF16: "bf16", FP8_E4M3: "fp8"}[_lib.kvq_layer_kv_dtype(window, skip_flags)]


# ---- device operations (torch tensors in, torch tensors out) -------------------------

def _torch():
    return _torch_mod


def _ptr(t):
    # a plain int: the c_void_p argtypes convert it without an extra Python object
    return None if t is None else t.data_ptr()


def _stream(stream=None, device=None):
    """Raw stream handle: ``stream`` if given, else torch's current stream of
    ``device`` (a torch.device of the call's tensors; the current device if None)."""
    if stream is not None:
        return stream.cuda_stream
    torch = _torch()
    idx = device.index if device is not None and device.index is not None \
        else torch.cuda.current_device()
    return torch._C._cuda_getCurrentRawStream(idx)


class PagedCache:
    """One layer's paged KV cache in the layout include/kvq.h fixes.

    fp8: k_pages uint8 [P][H][16][D] (token-major), v_pages uint8 [P][H][D][16]
    (dim-major), per-token-head scale pools float32 [P][H][16], or per-KV-head scale
    arrays float32 [H] (``k_head_scales`` / ``v_head_scales``, default 1.0).
    bf16: the same index orders with bfloat16 elements, no scales.
    """

    def __init__(self, num_pages: int, num_kv_heads: int, head_dim: int,
                 dtype: str = "fp8", mode: str = "per_token_head", device="cuda",
                 k_head_scales=None, v_head_scales=None):
        torch = _torch()
        self.num_pages, self.num_kv_heads, self.head_dim = num_pages, num_kv_heads, head_dim
        self.dtype, self.mode = dtype, mode
        el = torch.uint8 if dtype == "fp8" else torch.bfloat16
        self.k_pages = torch.zeros((num_pages, num_kv_heads, PAGE_SIZE, head_dim),
                                   dtype=el, device=device)
        self.v_pages = torch.zeros((num_pages, num_kv_heads, head_dim, PAGE_SIZE),
                                   dtype=el, device=device)
        if dtype == "fp8" and mode == "per_token_head":
            self.k_scales = torch.zeros((num_pages, num_kv_heads, PAGE_SIZE),
                                        dtype=torch.float32, device=device)
            self.v_scales = torch.zeros_like(self.k_scales)
        elif dtype == "fp8" and mode == "per_kv_head":
            def arr(x):
                t = torch.ones(num_kv_heads, dtype=torch.float32)
                if x is not None:
                    t[:] = torch.as_tensor(x, dtype=torch.float32).reshape(num_kv_heads)
                return t.to(device)
            self.k_scales, self.v_scales = arr(k_head_scales), arr(v_head_scales)
        else:
            self.k_scales = self.v_scales = None

    def desc(self) -> CacheDesc:
        """The C descriptor of the pools (built once: the pool tensors never move)."""
        d = getattr(self, "_desc", None)
        if d is None:
            d = self._desc = CacheDesc(
                _DTYPES[self.dtype], _MODES[self.mode], self.num_pages, PAGE_SIZE,
                self.num_kv_heads, self.head_dim,
                self.k_pages.data_ptr(), self.v_pages.data_ptr(),
                None if self.k_scales is None else self.k_scales.data_ptr(),
                None if self.v_scales is None else self.v_scales.data_ptr())
        return d

    @property
    def nbytes(self) -> int:
        n = self.k_pages.numel() * self.k_pages.element_size() * 2
        if self.k_scales is not None:
            n += self.k_scales.numel() * 4 * 2
        return n


def cache_write(cache: PagedCache, k, v, slot_mapping, k_scale: float = 1.0,
                v_scale: float = 1.0, token_stride: int = 0, stream=None) -> None:
    """k, v: bf16 [T][H][D] (or rows of ``token_stride`` elements); slot_mapping int64 [T]."""
    d = cache.desc()
    _check(_lib.kvq_cache_write(ctypes.byref(d), _ptr(k), _ptr(v), token_stride,
                                _ptr(slot_mapping), int(slot_mapping.numel()),
                                k_scale, v_scale, _stream(stream, k.device)), "cache_write")


def quantize_fp8(x, scale: float, out=None, stream=None):
    torch = _torch()
    if out is None:
        out = torch.empty(x.shape, dtype=torch.uint8, device=x.device)
    _check(_lib.kvq_quantize_fp8(_ptr(x), x.numel(), scale, _ptr(out), _stream(stream, x.device)),
           "quantize_fp8")
    return out


def decode_workspace_bytes(cache: PagedCache, num_seqs: int, num_q_heads: int,
                           max_seq_len: int, window: int = 0,
                           pages_per_split: int = 0) -> int:
    d = cache.desc()
    n = ctypes.c_size_t(0)
    _check(_lib.kvq_decode_workspace_bytes(ctypes.byref(d), num_seqs, num_q_heads,
                                           max_seq_len, window, pages_per_split,
                                           ctypes.byref(n)), "decode_workspace_bytes")
    return n.value


def decode_workspace(cache: PagedCache, num_seqs: int, num_q_heads: int,
                     max_seq_len: int, window: int = 0, pages_per_split: int = 0,
                     device="cuda"):
    """A zero-filled workspace of the size kvq_decode_workspace_bytes asks for (its
    completion counters must start at zero; calls leave them zero)."""
    torch = _torch()
    nb = decode_workspace_bytes(cache, num_seqs, num_q_heads, max_seq_len, window,
                                pages_per_split)
    return torch.zeros(max(nb, 256), dtype=torch.uint8, device=device)


def decode_attention(cache: PagedCache, q, block_table, seq_lens, max_seq_len: int,
                     scales: Scales | None = None, window: int = 0,
                     softmax_scale: float = 0.0, pages_per_split: int = 0,
                     out=None, out_dtype: str = "bf16", workspace=None, stream=None):
    """q bf16 [B][Hq][D]; block_table int32 [B][stride]; seq_lens int32 [B]."""
    torch = _torch()
    B, Hq, D = q.shape
    if scales is None:
        scales = Scales(1.0, 1.0, 1.0, 1.0)
    if out is None:
        out = torch.empty((B, Hq, D), dtype=torch.bfloat16 if out_dtype == "bf16"
                          else torch.float32, device=q.device)
    if workspace is None:
        workspace = decode_workspace(cache, B, Hq, max_seq_len, window, pages_per_split,
                                     q.device)
    d = cache.desc()
    _check(_lib.kvq_decode_attention(
        ctypes.byref(d), _ptr(q), B, Hq, _ptr(block_table), block_table.shape[1],
        _ptr(seq_lens), max_seq_len, ctypes.byref(scales), window, softmax_scale,
        pages_per_split, _ptr(out), _DTYPES[out_dtype], _ptr(workspace),
        workspace.numel(), _stream(stream, q.device)), "decode_attention")
    return out


def decode_attention_noalloc(cache: PagedCache, q, block_table, seq_lens, max_seq_len: int,
                             scales: Scales | None = None, window: int = 0,
                             softmax_scale: float = 0.0, pages_per_split: int = 0, out=None,
                             out_dtype: str = "bf16", stream=None):
    """decode_attention on the library's own device scratch (no workspace).  With
    ``out`` given, the call allocates nothing."""
    torch = _torch()
    B, Hq, D = q.shape
    if scales is None:
        scales = Scales(1.0, 1.0, 1.0, 1.0)
    if out is None:
        out = torch.empty((B, Hq, D), dtype=torch.bfloat16 if out_dtype == "bf16"
                          else torch.float32, device=q.device)
    d = cache.desc()
    _check(_lib.kvq_decode_attention_noalloc(
        ctypes.byref(d), _ptr(q), B, Hq, _ptr(block_table), block_table.shape[1],
        _ptr(seq_lens), max_seq_len, ctypes.byref(scales), window, softmax_scale,
        pages_per_split, _ptr(out), _DTYPES[out_dtype], _stream(stream, q.device)),
        "decode_attention_noalloc")
    return out


def decode_step(cache: PagedCache, q, k_new, v_new, block_table, seq_lens, max_seq_len: int,
                scales: Scales | None = None, window: int = 0, softmax_scale: float = 0.0,
                pages_per_split: int = 0, out=None, out_dtype: str = "bf16", workspace=None,
                stream=None):
    """Cache write of each sequence's new token (k_new, v_new bf16 [B][Hkv][D], stored at
    position seq_lens[b] - 1) and decode attention, in one launch."""
    torch = _torch()
    B, Hq, D = q.shape
    if scales is None:
        scales = Scales(1.0, 1.0, 1.0, 1.0)
    if out is None:
        out = torch.empty((B, Hq, D), dtype=torch.bfloat16 if out_dtype == "bf16"
                          else torch.float32, device=q.device)
    if workspace is None:
        workspace = decode_workspace(cache, B, Hq, max_seq_len, window, pages_per_split,
                                     q.device)
    d = cache.desc()
    _check(_lib.kvq_decode_step(
        ctypes.byref(d), _ptr(q), _ptr(k_new), _ptr(v_new), B, Hq, _ptr(block_table),
        block_table.shape[1], _ptr(seq_lens), max_seq_len, ctypes.byref(scales), window,
        softmax_scale, pages_per_split, _ptr(out), _DTYPES[out_dtype], _ptr(workspace),
        workspace.numel(), _stream(stream, q.device)), "decode_step")
    return out


def prefill_attention(cache: PagedCache, q, cu_q_lens, block_table, seq_lens,
                      max_q_len: int, scales: Scales | None = None, causal: bool = True,
                      window: int = 0, softmax_scale: float = 0.0, out=None,
                      out_dtype: str = "bf16", accumulation: str | None = None,
                      split: bool = True, workspace=None, stream=None):
    """q bf16 [Nq][Hq][D]; cu_q_lens int32 [B+1]; seq_lens int32 [B] (incl. new).

    accumulation: None (kvq_prefill_attention, or kvq_prefill_attention_ws with keys
    split over workgroups where the library asks for a workspace and `split` is set;
    `workspace`: a device uint8 tensor to use for it instead of a new one) or
    "mfma_chain" / "valu_add" (kvq_prefill_attention_accum with that level-2 form)."""
    torch = _torch()
    Nq, Hq, D = q.shape
    if scales is None:
        scales = Scales(1.0, 1.0, 1.0, 1.0)
    if out is None:
        out = torch.empty((Nq, Hq, D), dtype=torch.bfloat16 if out_dtype == "bf16"
                          else torch.float32, device=q.device)
    d = cache.desc()
    args = (ctypes.byref(d), _ptr(q), _ptr(cu_q_lens), int(seq_lens.numel()), Hq,
            _ptr(block_table), block_table.shape[1], _ptr(seq_lens), max_q_len,
            ctypes.byref(scales), int(causal), window, softmax_scale, _ptr(out),
            _DTYPES[out_dtype])
    if accumulation is None:
        # short query chunks on long contexts: keys split over workgroups through a
        # workspace (kvq_prefill_attention_ws) where the library asks for one
        nb = _lib.kvq_prefill_workspace_bytes(ctypes.byref(d), int(seq_lens.numel()), Hq,
                                              max_q_len) if split else 0
        if nb:
            ws = (torch.empty(nb, dtype=torch.uint8, device=q.device) if workspace is None
                  else workspace)
            _check(_lib.kvq_prefill_attention_ws(*args, _ptr(ws), ws.numel(),
                                                 _stream(stream, q.device)),
                   "prefill_attention_ws")
        else:
            _check(_lib.kvq_prefill_attention(*args, _stream(stream, q.device)),
                   "prefill_attention")
    else:
        _check(_lib.kvq_prefill_attention_accum(*args, ACCUMULATIONS[accumulation],
                                                _stream(stream, q.device)),
               "prefill_attention_accum")
    return out


def paged_logits(cache: PagedCache, q, cu_rows, row_lens, block_table, seq_lens,
                 out_len: int, scales: Scales | None = None, out=None, stream=None):
    """Query-key logits per query head: q bf16 [R][Hq][D]; cu_rows int32 [B+1];
    row_lens int32 [R]; seq_lens int32 [B] -> float32 [R][Hq][out_len] (out_len a
    multiple of 4), -inf past each row's visible length."""
    torch = _torch()
    R, Hq, D = q.shape
    if scales is None:
        scales = Scales(1.0, 1.0, 1.0, 1.0)
    if out is None:
        out = torch.empty((R, Hq, out_len), dtype=torch.float32, device=q.device)
    d = cache.desc()
    _check(_lib.kvq_paged_logits(
        ctypes.byref(d), _ptr(q), _ptr(cu_rows), int(seq_lens.numel()), R, Hq, _ptr(row_lens),
        _ptr(block_table), block_table.shape[1], _ptr(seq_lens), ctypes.byref(scales),
        _ptr(out), out.shape[2], _stream(stream, q.device)), "paged_logits")
    return out
