"""Host-side scale resolution and per-layer KV dtype policy (plain rules).

Test infrastructure only: see the package docstring for who may import it.

Source: "[vLLM] KV Cache Quantization: KV cache FP8/INT8 quantization"
(blog.secrett2633.cloud), sections "BaseKVCacheMethod", "Per-Token-Head vs
Per-Tensor quantization", "Q/Prob scales and FP8 attention" and "Scale merging
logic"; and "vLLM FP8 KV-Cache and Attention Quantization Update", section "Hybrid
attention and layer skipping" (``--kv-cache-dtype-skip-layers sliding_window``).

Rules as the pages state them:
  * every scale parameter starts at the sentinel -1.0, meaning "not loaded";
  * per-token-head mode: the kernel computes K/V scales at store time, the
    per-tensor K/V scales are set to 1.0 and the Q/prob parameters are dropped
    (so both act as 1.0);
  * per-tensor mode: k > 0 and v > 0 -> use them; k < 0 and v < 0 -> both 1.0;
    otherwise a single kv scale was loaded into k: k must be positive and both
    become max(k, v);
  * q_scale > 0 -> use it, else 1.0.  The page shows no rule for prob_scale;
    reading: the same rule as q_scale;
  * an fp8 cache used with q_scale == 1.0 or prob_scale == 1.0 raises a one-time
    "uncalibrated" warning;
  * the platform-specific doubling of K/V scales for the FNUZ fp8 variant is not
    applied: the target's fp8 type is the OCP e4m3 format;
  * per-KV-head scale arrays ("vLLM FP8 KV-Cache and Attention Quantization
    Update", section "Kernel and fusion optimizations": one scale per KV head):
    the pages give no loading rule; reading: each head's (k, v) pair follows the
    per-tensor rules.

Skip policy: a layer keeps a bf16 cache iff the sliding-window skip flag is set and
the layer has a window (> 0); every other layer uses the fp8 cache.
"""
from __future__ import annotations

from dataclasses import dataclass

SENTINEL = -1.0
WARN_UNCALIBRATED_Q_OR_PROB = 1
SKIP_SLIDING_WINDOW = 1


class ScaleError(ValueError):
    pass


@dataclass(frozen=True)
class Scales:
    q_scale: float
    k_scale: float
    v_scale: float
    prob_scale: float


def resolve(mode: str, k: float, v: float, q: float, prob: float):
    """Resolve raw (possibly sentinel) scales.  Returns (Scales, warn_flags)."""
    if mode == "per_token_head":
        # the page's early return: no per-tensor checks and no warning
        return Scales(1.0, 1.0, 1.0, 1.0), 0
    if mode not in ("per_tensor", "per_kv_head"):
        raise ScaleError(mode)
    # per_kv_head: the per-tensor rules for one KV head's (k, v) pair
    if k > 0.0 and v > 0.0:
        ks, vs = k, v
    elif k < 0.0 and v < 0.0:
        ks = vs = 1.0
    else:
        if not k > 0.0:
            raise ScaleError("a single kv scale must be loaded into k_scale")
        ks = vs = max(k, v)
    qs = q if q > 0.0 else 1.0
    ps = prob if prob > 0.0 else 1.0
    warn = WARN_UNCALIBRATED_Q_OR_PROB if (qs == 1.0 or ps == 1.0) else 0
    return Scales(qs, ks, vs, ps), warn


def layer_kv_dtype(window: int, skip_flags: int) -> str:
    """"bf16" for a sliding-window layer when the sliding-window skip flag is set,
    else "fp8"."""
    if (skip_flags & SKIP_SLIDING_WINDOW) and window > 0:
        return "bf16"
    return "fp8"
