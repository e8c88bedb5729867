"""kvq: FP8 (e4m3) paged KV-cache attention for AMD MI355X (gfx950).

The compute lives in libkvq.so (hand-written HIP kernels behind the C ABI of
include/kvq.h); this package is its thin Python binding.  Importing it fails when
the library is not built: there is no CPU or PyTorch fallback.
"""
from .binding import (  # noqa: F401
    BF16, DECODE_COUNTER_BYTES, DECODE_MAX_SPLIT_UNITS, DECODE_SCRATCH_BYTES, F32, FP8_E4M3, PAGE_SIZE, PER_KV_HEAD, PER_TENSOR, PER_TOKEN_HEAD,
    SKIP_SLIDING_WINDOW, WARN_UNCALIBRATED_Q_OR_PROB, CacheDesc, KvqError, PagedCache, Scales, abi_version,
    cache_write, decode_attention, decode_attention_noalloc, decode_step, decode_workspace, decode_workspace_bytes,
    exported, header_functions,
    last_error, layer_kv_dtype, paged_logits, prefill_attention, quantize_fp8, resolve_scales,
    status_string,
)
