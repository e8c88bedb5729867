"""Helpers for the GPU parity tests: move seeded inputs to the device, fill caches
through the library, read device pools back in the oracle's logical layout, and
build the oracle's reference for the same inputs.

Nothing here computes any part of the method: device results come from libkvq.so,
expected values from ``oracle``.
"""
from __future__ import annotations

import sys

import numpy as np
import torch

import workloads
from oracle import attention, cache as ocache

# Acceptance bar of the attention outputs against the float64 oracle computed from
# the same dequantised cache: |o - O| <= ATOL + RTOL * |O| elementwise.
ATOL = 5e-3
RTOL = 2e-2
# Second bar: against the float64 attention over the raw (unquantised) bf16 Q/K/V,
# |o - O_bf16| <= BF16_TOL + BF16_TOL * |O_bf16| elementwise.
BF16_TOL = 6e-2


def log(*a):
    print(*a, flush=True, file=sys.stderr)


def dev_bf16(x_f32: np.ndarray) -> torch.Tensor:
    """float32 numpy array of bf16 values -> bf16 device tensor with the same bits."""
    bits = workloads.bf16_bits(x_f32).view(np.int16)
    return torch.from_numpy(np.ascontiguousarray(bits)).view(torch.bfloat16).cuda()


def dev(x, dtype=None) -> torch.Tensor:
    t = torch.from_numpy(np.ascontiguousarray(x))
    if dtype is not None:
        t = t.to(dtype)
    return t.cuda()


def write_cache(kvq, case, dtype="fp8", mode="per_token_head", k_scale=1.0, v_scale=1.0,
                rows=None, chunk=1 << 20):
    """Allocate a device cache for ``case`` and write every token (or ``rows``)
    through kvq.cache_write, in chunks of tokens.  per_kv_head: k_scale / v_scale are
    the per-head arrays (the cache's scale arrays; the call's scalars are unused)."""
    if mode == "per_kv_head":
        c = kvq.PagedCache(case.num_pages, case.num_kv_heads, case.head_dim, dtype, mode,
                           k_head_scales=k_scale, v_head_scales=v_scale)
        k_scale = v_scale = 1.0
    else:
        c = kvq.PagedCache(case.num_pages, case.num_kv_heads, case.head_dim, dtype, mode)
    idx = np.arange(len(case.k)) if rows is None else np.asarray(rows)
    per_tok = case.num_kv_heads * case.head_dim
    step = max(1, chunk // per_tok)
    for i in range(0, len(idx), step):
        sel = idx[i:i + step]
        kvq.cache_write(c, dev_bf16(case.k[sel]), dev_bf16(case.v[sel]),
                        dev(case.slots[sel].astype(np.int64)), k_scale, v_scale)
    return c


def read_pools(c):
    """Device pools -> numpy in the oracle's logical layout [P][H][16][D]."""
    k = c.k_pages.cpu()
    v = c.v_pages.cpu().transpose(2, 3).contiguous()
    if c.dtype == "fp8":
        out = {"k_codes": k.numpy(), "v_codes": v.numpy()}
        if c.k_scales is not None and c.mode == "per_token_head":
            out["k_scales"] = c.k_scales.cpu().numpy()
            out["v_scales"] = c.v_scales.cpu().numpy()
        return out
    return {"k": k.float().numpy(), "v": v.float().numpy()}


def oracle_pools(case, mode="per_token_head", k_scale=1.0, v_scale=1.0, rows=None):
    pools = ocache.new_pools(case.num_pages, case.num_kv_heads, case.head_dim)
    idx = np.arange(len(case.k)) if rows is None else np.asarray(rows)
    ocache.cache_write(pools, case.k[idx], case.v[idx], case.slots[idx], mode,
                       k_scale, v_scale)
    return pools


def oracle_pools_for_heads(case, b, kv_heads, mode, k_scale=1.0, v_scale=1.0):
    """Logical float64 K/V pools restricted to sequence b and some KV heads (other
    entries zero): enough for the oracle's attention of those heads."""
    sel = np.nonzero(case.token_seq == b)[0]
    P, D = case.num_pages, case.head_dim
    kp = np.zeros((P, case.num_kv_heads, 16, D))
    vp = np.zeros_like(kp)
    page, off = case.slots[sel] // 16, case.slots[sel] % 16
    for g in kv_heads:
        for name, x, ts, dst in (("k", case.k, k_scale, kp), ("v", case.v, v_scale, vp)):
            codes, s = ocache.quantize_rows(x[sel, g], mode, ts)
            dst[page, g, off] = ocache.dequantize(codes, s[:, None])
    return kp, vp


def assert_close_to_oracle(got, want, what=""):
    err = np.abs(got - want)
    bound = ATOL + RTOL * np.abs(want)
    bad = err > bound
    if bad.any():
        i = np.unravel_index(np.argmax(err - bound), err.shape)
        raise AssertionError(
            f"{what}: {int(bad.sum())}/{bad.size} outside {ATOL}+{RTOL}|O|; worst at "
            f"{i}: got {got[i]!r} want {want[i]!r} (max abs err {err.max():.3g})")
    return float(err.max())


def raw_pools_for_heads(case, b, kv_heads):
    """Logical float64 K/V pools of sequence b's raw bf16 rows for some KV heads (other
    entries zero): the inputs of the bf16-cache reference."""
    sel = np.nonzero(case.token_seq == b)[0]
    P, D = case.num_pages, case.head_dim
    kp = np.zeros((P, case.num_kv_heads, 16, D))
    vp = np.zeros_like(kp)
    page, off = case.slots[sel] // 16, case.slots[sel] % 16
    for g in kv_heads:
        kp[page, g, off] = case.k[sel, g]
        vp[page, g, off] = case.v[sel, g]
    return kp, vp


def check_bf16_bar(got, want_bf16, want_exact=None, what="", require=True):
    """The second bar.  With require=False (a workload where the oracle's own exact
    result already misses it) the device's distance to O_bf16 must instead stay
    within the first bar of the oracle's own distance, element by element:
    |o - O_bf16| <= |O_exact - O_bf16| + ATOL + RTOL * |O_exact|.  Returns the
    fraction of elements within the bar for the device (and for the oracle)."""
    err = np.abs(got - want_bf16)
    lim = BF16_TOL + BF16_TOL * np.abs(want_bf16)
    frac = float(np.mean(err <= lim))
    frac_oracle = None
    if want_exact is not None:
        frac_oracle = float(np.mean(np.abs(want_exact - want_bf16) <= lim))
    log(f"  {what}: within {BF16_TOL} of the bf16-cache result: device {frac:.4f}"
        + ("" if frac_oracle is None else f", oracle's exact result {frac_oracle:.4f}"))
    if require:
        bad = err > lim
        if bad.any():
            i = np.unravel_index(np.argmax(err - lim), err.shape)
            raise AssertionError(f"{what}: {int(bad.sum())}/{bad.size} outside {BF16_TOL} "
                                 f"of the bf16 result; worst got {got[i]!r} "
                                 f"want {want_bf16[i]!r}")
    else:
        assert want_exact is not None
        slack = np.abs(want_exact - want_bf16) + ATOL + RTOL * np.abs(want_exact)
        assert np.all(err <= slack), what
    return frac, frac_oracle
