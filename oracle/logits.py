"""Paged query-key logits in float64 over a dequantised cache (plain definition).

Test infrastructure only: see the package docstring for who may import it.

What it computes ("vLLM Qwen3.8-Flash-Next: QSA Indexer ... FP8 support" page, section
on tests/models/qwen4_exp/test_qsa_reference.py): a sparse-attention indexer scores
every cache token a query row may see, from an FP8 (or bf16) paged cache, and its
top-k selection reads those scores; with FP8 the scores are compared value by value
(no reduced-precision accumulation on exact-fp32 hardware).  For query row r of
request b (cu_rows[b] <= r < cu_rows[b + 1]) and query head h, with key head
g = h // (Hq / Hkv) and key j of request b fetched through its block table (token j in
physical page block_table[b][j // 16] at offset j % 16):

    logits[r][h][j] = q[r][h] . k_j[g]      for j < row_lens[r]
    logits[r][h][j] = -inf                  for row_lens[r] <= j < out_len
(only keys j < out_len are represented: a narrower output holds a prefix).

Readings where the page is silent: the scores stay per query head (the page does not
say how the indexer's heads are combined, so that reduction and the top-k rule are
the caller's); no softmax scale is applied (raw q . k); a row sees the first
row_lens[r] keys of its request (decode rows: the whole cache; chunked-prefill rows:
the causal prefix).  The query is the dequantised e4m3 query (q_scale times its code)
for an FP8 cache and the bf16 query itself for a bf16 cache, like the attention paths.
"""
from __future__ import annotations

import numpy as np

from .attention import gather


def paged_logits(q, cu_rows, row_lens, k_pool, block_table, out_len: int) -> np.ndarray:
    """q [R][Hq][D] (float), cu_rows [B + 1], row_lens [R], k_pool [P][Hkv][16][D]
    (dequantised values), block_table [B][max_pages] -> float64 [R][Hq][out_len]."""
    q = np.asarray(q, np.float64)
    R, Hq, D = q.shape
    Hkv = k_pool.shape[1]
    group = Hq // Hkv
    out = np.full((R, Hq, out_len), -np.inf, np.float64)
    cu_rows = np.asarray(cu_rows, np.int64)
    row_lens = np.asarray(row_lens, np.int64)
    for b in range(len(cu_rows) - 1):
        r0, r1 = int(cu_rows[b]), int(cu_rows[b + 1])
        if r1 <= r0:
            continue
        n_keys = min(int(row_lens[r0:r1].max()), out_len)  # only keys j < out_len exist
        if n_keys <= 0:
            continue
        k = np.asarray(gather(k_pool, block_table[b], n_keys), np.float64)  # [L][Hkv][D]
        for r in range(r0, r1):
            n = min(int(row_lens[r]), out_len)
            for h in range(Hq):
                out[r, h, :n] = k[:n, h // group, :] @ q[r, h]
    return out
