"""Quantising cache write: scales, codes, paged scatter (plain CPU definition).

Test infrastructure only: see the package docstring for who may import it.

Sources.
  * "[vLLM] KV Cache Quantization: KV cache FP8/INT8 quantization"
    (blog.secrett2633.cloud), section "Per-Token-Head vs Per-Tensor quantization":
    per-tensor mode uses one K and one V scale for the whole layer (from the
    checkpoint, else 1.0); per-token-head mode computes a separate scale for every
    (token, head) in the kernel at the moment the cache is stored, needing no
    checkpoint scale.
  * "vLLM FP8 KV-Cache and Attention Quantization Update", section "Kernel and
    fusion optimizations": scale arrays with one scale per KV head (per-KV-head
    mode: per-tensor quantisation with the head's own scale).
  * The per-token-head scale is amax / 448 and the code is
    clamp(round_rne(v / scale), +-448).
  * Pages and block tables: "vLLM Qwen3.8-Flash-Next: FP8 support for the QSA
    indexer cache", section "Code analysis" (page size 16, a random permutation of
    pages as the page table).

Readings where the pages are silent (each one is also listed in the design notes):
  * the quotient v / scale is one IEEE float32 division, then the e4m3 rounding
    (double rounding, as a device computing in float32 does);
  * a zero row (amax = 0) gets scale 1.0 and all-zero codes (1.0 is the pages'
    default scale); amax propagates NaN, so a row holding a NaN gets a NaN scale;
  * a NaN quotient encodes as 0x7F with the sign bit of v (the sign of a NaN
    produced by a division is not fixed by IEEE, the sign of v is);
  * slot = page * page_size + offset; a negative slot means "do not store".

Logical cache layout used by the oracle: codes[page][kv_head][offset][dim] and
scales[page][kv_head][offset] for K and for V alike.  The device's physical layout
is a separate matter, handled by the tests that read device pools.
"""
from __future__ import annotations

import numpy as np

from . import e4m3

PAGE_SIZE = 16


def per_token_head_scale(x) -> np.ndarray:
    """float32 scale per row of ``x`` (rows along the last axis): fl32(amax / 448)."""
    x = np.asarray(x, dtype=np.float32)
    with np.errstate(invalid="ignore"):
        amax = np.max(np.abs(x), axis=-1)  # exact; NaN propagates
        s = amax.astype(np.float32) / np.float32(e4m3.E4M3_MAX)
    return np.where(amax == 0, np.float32(1.0), s).astype(np.float32)


def quantize(x, scale) -> np.ndarray:
    """Codes of ``x`` at ``scale`` (broadcast against x): enc(fl32(x / scale))."""
    x = np.asarray(x, dtype=np.float32)
    s = np.asarray(scale, dtype=np.float32)
    with np.errstate(invalid="ignore", divide="ignore", over="ignore"):
        qt = (x / s).astype(np.float32)
    flat = qt.reshape(-1)
    codes = np.empty(flat.shape, np.uint8)
    step = 1 << 16   # cache-sized temporaries; the arithmetic is elementwise
    for i in range(0, flat.size, step):
        codes[i:i + step] = e4m3.encode(flat[i:i + step])
    codes = codes.reshape(qt.shape)
    nan_q = np.isnan(qt)
    nan_code = np.where(np.signbit(x), 0xFF, 0x7F).astype(np.uint8)
    return np.where(nan_q, nan_code, codes).astype(np.uint8)


def dequantize(codes, scale) -> np.ndarray:
    """float64 values val(code) * scale (exact: 4 x 24 significant bits < 53)."""
    return e4m3.decode(codes) * np.asarray(scale, dtype=np.float64)


def quantize_rows(x, mode: str, tensor_scale: float = 1.0):
    """Quantise rows of D values.  Returns (codes uint8 [..., D], scales float32 [...]).

    mode "per_tensor": every row uses ``tensor_scale``.
    mode "per_kv_head": ``x`` is [..., Hkv, D]; rows of head h use tensor_scale[h].
    mode "per_token_head": every row uses its own amax / 448.
    """
    x = np.asarray(x, dtype=np.float32)
    if mode == "per_tensor":
        s = np.full(x.shape[:-1], tensor_scale, dtype=np.float32)
    elif mode == "per_kv_head":
        s = np.broadcast_to(np.asarray(tensor_scale, np.float32), x.shape[:-1]).copy()
    elif mode == "per_token_head":
        s = per_token_head_scale(x)
    else:
        raise ValueError(mode)
    return quantize(x, s[..., None]), s


def new_pools(num_pages: int, num_kv_heads: int, head_dim: int):
    """Empty logical FP8 cache: dict of K/V codes and scales (codes 0, scales NaN)."""
    shape = (num_pages, num_kv_heads, PAGE_SIZE, head_dim)
    return {
        "k_codes": np.zeros(shape, np.uint8),
        "v_codes": np.zeros(shape, np.uint8),
        "k_scales": np.full(shape[:3], np.nan, np.float32),
        "v_scales": np.full(shape[:3], np.nan, np.float32),
    }


def cache_write(pools, k, v, slot_mapping, mode: str, k_scale=1.0, v_scale=1.0) -> None:
    """Quantise K/V rows of T tokens ([T][Hkv][D], float32 values of bf16) into pools.

    Token t goes to page slot_mapping[t] // 16, offset slot_mapping[t] % 16; tokens
    whose slot is negative are skipped.  k_scale / v_scale: a float (per_tensor) or
    one float per KV head (per_kv_head); every stored row records its scale in the
    pools' per-slot scales, so dequantisation reads the same way in every mode.
    """
    slots = np.asarray(slot_mapping, dtype=np.int64)
    keep = slots >= 0
    page, off = slots[keep] // PAGE_SIZE, slots[keep] % PAGE_SIZE
    for name, x, ts in (("k", k, k_scale), ("v", v, v_scale)):
        codes, s = quantize_rows(np.asarray(x, np.float32)[keep], mode, ts)
        pools[name + "_codes"][page, :, off, :] = codes
        pools[name + "_scales"][page, :, off] = s


def dequantized(pools, which: str) -> np.ndarray:
    """float64 [P][Hkv][16][D] dequantised K or V pool."""
    return dequantize(pools[which + "_codes"], pools[which + "_scales"][..., None])


def quantize_q(q, q_scale: float):
    """Query quantisation: codes = enc(fl32(q / q_scale)); q_hat = val(code) * q_scale.

    "[vLLM] KV Cache Quantization", section "Q/Prob scales and FP8 attention": FP8
    attention needs a scale for Q (and for the softmax probabilities).
    """
    codes = quantize(np.asarray(q, np.float32), np.float32(q_scale))
    return codes, dequantize(codes, np.float32(q_scale))
