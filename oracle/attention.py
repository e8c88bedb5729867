"""Paged GQA softmax attention in float64 over a dequantised cache (plain definition).

Test infrastructure only: see the package docstring for who may import it.

What it computes.  For a query row q of head h the key head is g = h // (Hq / Hkv)
(contiguous groups; the pages leave the mapping open).  Over the visible keys j:
    s_j = (q . k_j) * sm_scale,   sm_scale = 1 / sqrt(D) unless given,
    o   = sum_j softmax(s)_j * v_j      (maximum subtracted before exp).
Keys are fetched through the block table: token j of sequence b lives in physical
page block_table[b][j // 16] at offset j % 16.

Visibility (readings where the pages are silent):
  * decode: the query is the sequence's last token; keys 0 .. seq_len-1 (the cache
    write of the current token comes first, so seq_len counts it); with a window
    W > 0 only the last W keys, the current one included ("vLLM FP8 KV-Cache and
    Attention Quantization Update", section "Hybrid attention and layer skipping":
    sliding windows of e.g. 128 tokens);
  * chunked prefill: the n new queries of a sequence sit at absolute positions
    ctx .. ctx+n-1 with ctx = seq_len - n; query i sees keys 0 .. ctx+i (causal,
    bottom-right aligned), and with W > 0 only keys > ctx+i-W.
  * a sequence with seq_len = 0 gives a zero output row.

Precision: the pages' two-level accumulation exists because low-precision
accumulation loses accuracy once the contraction reaches 100k+ keys; this oracle
sidesteps that entirely by working in float64 throughout.
"""
from __future__ import annotations

import math

import numpy as np

PAGE_SIZE = 16
LOG2E = 1.0 / math.log(2.0)


def gather(pool, block_table_row, n_tokens: int) -> np.ndarray:
    """Logical token rows [n_tokens][Hkv][D] of one sequence from a paged pool
    [P][Hkv][16][D]."""
    j = np.arange(n_tokens)
    pages = np.asarray(block_table_row, dtype=np.int64)[j // PAGE_SIZE]
    return pool[pages, :, j % PAGE_SIZE, :]


def attend_rows(q, k, v, lo, hi, sm_scale: float, spread: bool = False,
                weight_error=None):
    """Softmax attention of query rows q [R][D] over rows k, v [L][D].

    Row r sees keys lo[r] .. hi[r] inclusive; an empty range gives zeros.

    With ``spread`` also returns, per row and channel, the attention-weighted mean
    absolute deviation of V from the output, sum_j w_j |v_j - o|: the amount by
    which the output moves per unit of relative error in the weights (if every
    weight w_j becomes w_j (1 + e_j) with |e_j| <= r, renormalised, the output
    moves by at most r / (1 - r) times this).

    With ``weight_error`` (a function of (gap, j) giving, for key j of a row whose
    log2-domain score lies ``gap`` = (s_j - max_i s_i) * log2(e) <= 0 below the row's
    largest, a bound e_j in [0, 1] on the relative error of that key's weight) the
    second result is instead the largest move of the renormalised weighted mean under
    those errors:  sum_j e_j w_j |v_j - o| / sum_j w_j (1 - e_j).  (Exact: with
    w'_j = w_j (1 + d_j), o' - o = sum_j w_j d_j (v_j - o) / sum_j w'_j, because
    sum_j w_j (v_j - o) = 0.)  Infinite when the denominator is not positive.
    """
    q = np.asarray(q, np.float64)
    k = np.asarray(k, np.float64)
    v = np.asarray(v, np.float64)
    out = np.zeros((q.shape[0], v.shape[1]), np.float64)
    dev = np.zeros_like(out)
    if k.shape[0] == 0:
        return (out, dev) if (spread or weight_error is not None) else out
    s = (q @ k.T) * sm_scale                      # [R][L]
    j = np.arange(k.shape[0])[None, :]
    vis = (j >= np.asarray(lo)[:, None]) & (j <= np.asarray(hi)[:, None])
    s = np.where(vis, s, -np.inf)
    m = np.max(s, axis=1, keepdims=True)
    ok = np.isfinite(m[:, 0])
    m = np.where(np.isfinite(m), m, 0.0)
    p = np.where(vis, np.exp(s - m), 0.0)
    l = p.sum(axis=1, keepdims=True)
    o = (p @ v) / np.where(l > 0, l, 1.0)
    out[ok] = o[ok]
    if not spread and weight_error is None:
        return out
    for r in np.nonzero(ok)[0]:
        if weight_error is None:
            dev[r] = (p[r] @ np.abs(v - o[r])) / l[r, 0]
            continue
        js = np.nonzero(vis[r])[0]
        gap = (s[r, js] - m[r, 0]) * LOG2E
        e = np.clip(np.asarray(weight_error(gap, js), np.float64), 0.0, 1.0)
        den = p[r, js] @ (1.0 - e)
        dev[r] = ((p[r, js] * e) @ np.abs(v[js] - o[r])) / den if den > 0 else np.inf
    return out, dev


def default_sm_scale(head_dim: int) -> float:
    return 1.0 / math.sqrt(head_dim)


def decode(q, k_pool, v_pool, block_table, seq_lens, window: int = 0,
           sm_scale: float | None = None, heads=None) -> np.ndarray:
    """Decode attention.  q [B][Hq][D]; pools [P][Hkv][16][D] (float64 values).

    Returns float64 [B][Hq][D].  ``heads`` optionally restricts the work to a list
    of (b, h) pairs (other rows are left at zero), for sampled checks at full size.
    """
    q = np.asarray(q, np.float64)
    B, Hq, D = q.shape
    Hkv = k_pool.shape[1]
    G = Hq // Hkv
    sm = default_sm_scale(D) if sm_scale is None else sm_scale
    out = np.zeros((B, Hq, D), np.float64)
    want = None if heads is None else set(map(tuple, heads))
    for b in range(B):
        L = int(seq_lens[b])
        if L == 0:
            continue
        lo = max(0, L - window) if window > 0 else 0
        need = [h for h in range(Hq) if want is None or (b, h) in want]
        if not need:
            continue
        kv_heads = sorted({h // G for h in need})
        k = gather(k_pool[:, kv_heads], block_table[b], L)
        v = gather(v_pool[:, kv_heads], block_table[b], L)
        for h in need:
            gi = kv_heads.index(h // G)
            out[b, h] = attend_rows(q[b, h][None, :], k[lo:, gi], v[lo:, gi],
                                    [0], [L - 1 - lo], sm)[0]
    return out


def prefill(q, cu_q_lens, k_pool, v_pool, block_table, seq_lens, causal: bool = True,
            window: int = 0, sm_scale: float | None = None, rows=None,
            spread: bool = False, weight_error=None):
    """Chunked-prefill attention.  q [Nq][Hq][D] holds the new queries of all
    sequences back to back (sequence b owns rows cu_q_lens[b] .. cu_q_lens[b+1]-1).

    Returns float64 [Nq][Hq][D].  ``rows`` optionally restricts the work to a sorted
    list of query row indices (other rows stay zero).  With ``spread`` also returns
    attend_rows' weighted mean absolute deviation of V, same shape.  With
    ``weight_error`` (a function of (b, g) returning attend_rows' per-key function for
    sequence b, KV head g; keys j are the sequence's positions) the second result is
    attend_rows' bound under those per-key weight errors instead.
    """
    q = np.asarray(q, np.float64)
    Nq, Hq, D = q.shape
    Hkv = k_pool.shape[1]
    G = Hq // Hkv
    sm = default_sm_scale(D) if sm_scale is None else sm_scale
    out = np.zeros((Nq, Hq, D), np.float64)
    dev = np.zeros_like(out)
    for b in range(len(seq_lens)):
        r0, r1 = int(cu_q_lens[b]), int(cu_q_lens[b + 1])
        n, L = r1 - r0, int(seq_lens[b])
        if n == 0 or L == 0:
            continue
        ctx = L - n
        idx = np.arange(r0, r1) if rows is None else np.asarray(
            [r for r in rows if r0 <= r < r1], dtype=np.int64)
        if idx.size == 0:
            continue
        pos = ctx + (idx - r0)                     # absolute query positions
        hi = pos if causal else np.full_like(pos, L - 1)
        lo = np.maximum(0, pos - window + 1) if window > 0 else np.zeros_like(pos)
        k = gather(k_pool, block_table[b], L)
        v = gather(v_pool, block_table[b], L)
        for h in range(Hq):
            g = h // G
            we = None if weight_error is None else weight_error(b, g)
            res = attend_rows(q[idx, h], k[:, g], v[:, g], lo, hi, sm, spread, we)
            if spread or we is not None:
                out[idx, h], dev[idx, h] = res
            else:
                out[idx, h] = res
    return (out, dev) if (spread or weight_error is not None) else out
