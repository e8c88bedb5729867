"""Seeded synthetic inputs for FP8 paged-attention workloads.

Shared by the tests, the benchmark and the smoke check: both the CPU oracle and the
device path are fed from here.  This package holds none of the method's arithmetic
(no quantisation, scaling or attention): it draws normal variates, rounds them to
bfloat16 input values, and lays out block tables, slot mappings and lengths.

Input recipe (one fixed seed per workload; draws happen in this order: Q, K, V,
outlier channels, planted position, block-table permutation):
  * values are float32 standard normals from numpy's PCG64 generator, times the
    workload's standard deviation, rounded to bfloat16 by round-to-nearest-even;
  * "outliers": per tensor (K, V) and KV head, 4 distinct channel indices drawn
    once and shared by all tokens, whose values are multiplied by 20 before the
    bfloat16 rounding;
  * "planted key": at one seeded position, in every KV head g, the key row is
    8 * q / |q| with q the query of the group's first head (h = g * G) -- the decode
    query, or the last new row of a prefill chunk -- rounded to bfloat16;
  * block tables: identity (sequence b owns pages b*P .. b*P+P-1) or a seeded
    permutation of all pages reshaped to [B][P], as the pages' tests build them.
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np

PAGE_SIZE = 16


def bf16_round(x) -> np.ndarray:
    """float32 -> nearest bfloat16 value (ties to even), returned as float32."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    u = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return (u.astype(np.uint32) << 16).view(np.float32)


def bf16_bits(x) -> np.ndarray:
    """uint16 bit patterns of float32 values that are already bfloat16 values."""
    return (np.ascontiguousarray(x, dtype=np.float32).view(np.uint32) >> 16).astype(
        np.uint16)


def normal_bf16(rng: np.random.Generator, shape, std: float = 1.0) -> np.ndarray:
    x = rng.standard_normal(size=shape, dtype=np.float32)
    if std != 1.0:
        x *= np.float32(std)
    return bf16_round(x)


@dataclass
class DecodeCase:
    """Inputs of one decode step over a paged cache.

    q:   [B][Hq][D]        bf16 values (float32 arrays)
    k,v: [T][Hkv][D]       all tokens of all sequences, sequence-major
    token_seq, token_pos:  [T] owning sequence and position of every token row
    slots: [T] int64       physical slot of every token row
    block_table: [B][max_pages] int32, seq_lens: [B] int32
    """
    name: str
    q: np.ndarray
    k: np.ndarray
    v: np.ndarray
    token_seq: np.ndarray
    token_pos: np.ndarray
    slots: np.ndarray
    block_table: np.ndarray
    seq_lens: np.ndarray
    num_pages: int
    num_kv_heads: int
    head_dim: int
    window: int = 0
    meta: dict = field(default_factory=dict)

    @property
    def num_q_heads(self) -> int:
        return self.q.shape[1]

    def last_token_rows(self) -> np.ndarray:
        """Row indices (into k/v) of the current (last) token of every non-empty
        sequence."""
        ends = np.cumsum(self.seq_lens.astype(np.int64))
        return (ends - 1)[self.seq_lens > 0]


def make_block_table(rng, num_seqs: int, pages_per_seq: int, kind: str,
                     num_pages: int | None = None) -> np.ndarray:
    total = num_seqs * pages_per_seq
    if kind == "identity":
        return np.arange(total, dtype=np.int32).reshape(num_seqs, pages_per_seq)
    if kind == "perm":
        n = total if num_pages is None else num_pages
        return rng.permutation(n)[:total].astype(np.int32).reshape(
            num_seqs, pages_per_seq)
    raise ValueError(kind)


def token_layout(seq_lens, block_table):
    """Sequence/position/slot of every token row, sequence-major."""
    seq_lens = np.asarray(seq_lens, np.int64)
    token_seq = np.repeat(np.arange(len(seq_lens)), seq_lens)
    starts = np.concatenate([[0], np.cumsum(seq_lens)[:-1]])
    token_pos = np.arange(int(seq_lens.sum())) - starts[token_seq]
    pages = block_table[token_seq, token_pos // PAGE_SIZE].astype(np.int64)
    slots = pages * PAGE_SIZE + token_pos % PAGE_SIZE
    return token_seq, token_pos, slots


def make_decode_case(seed: int, seq_lens, num_q_heads: int, num_kv_heads: int,
                     head_dim: int, table: str = "perm", std: float = 1.0,
                     outliers: int = 0, planted: bool = False, window: int = 0,
                     extra_pages: int = 0, name: str = "case") -> DecodeCase:
    """General seeded decode case (every config below is one of these)."""
    rng = np.random.default_rng(seed)
    seq_lens = np.asarray(seq_lens, dtype=np.int32)
    B = len(seq_lens)
    T = int(seq_lens.sum())
    q = normal_bf16(rng, (B, num_q_heads, head_dim))
    k = rng.standard_normal(size=(T, num_kv_heads, head_dim), dtype=np.float32)
    v = rng.standard_normal(size=(T, num_kv_heads, head_dim), dtype=np.float32)
    if std != 1.0:
        k *= np.float32(std)
        v *= np.float32(std)
    meta = {}
    if outliers:
        for name_, x in (("k", k), ("v", v)):
            ch = np.stack([rng.choice(head_dim, size=outliers, replace=False)
                           for _ in range(num_kv_heads)])
            meta[name_ + "_outlier_channels"] = ch
            for g in range(num_kv_heads):
                x[:, g, ch[g]] *= np.float32(20.0)
    k = bf16_round(k)
    v = bf16_round(v)
    pages_per_seq = max(1, -(-int(seq_lens.max()) // PAGE_SIZE)) if B else 1
    if planted:
        G = num_q_heads // num_kv_heads
        pos = int(rng.integers(0, int(seq_lens.min())))
        meta["planted_pos"] = pos
        starts = np.concatenate([[0], np.cumsum(seq_lens)[:-1]])
        for b in range(B):
            for g in range(num_kv_heads):
                qv = q[b, g * G].astype(np.float64)
                k[starts[b] + pos, g] = bf16_round(
                    (8.0 * qv / np.linalg.norm(qv)).astype(np.float32))
    num_pages = B * pages_per_seq + extra_pages
    bt = make_block_table(rng, B, pages_per_seq, table, num_pages)
    ts, tp, slots = token_layout(seq_lens, bt)
    return DecodeCase(name, q, k, v, ts, tp, slots, bt, seq_lens, num_pages,
                      num_kv_heads, head_dim, window, meta)


@dataclass
class PrefillCase:
    """Inputs of one chunked-prefill step.

    q: [Nq][Hq][D] new queries (all sequences back to back), cu_q_lens [B+1];
    k, v, token_* and slots cover every token (cached and new) as in DecodeCase;
    seq_lens counts the new tokens.
    """
    name: str
    q: np.ndarray
    cu_q_lens: np.ndarray
    k: np.ndarray
    v: np.ndarray
    token_seq: np.ndarray
    token_pos: np.ndarray
    slots: np.ndarray
    block_table: np.ndarray
    seq_lens: np.ndarray
    num_pages: int
    num_kv_heads: int
    head_dim: int
    window: int = 0
    meta: dict = field(default_factory=dict)

    def new_token_rows(self) -> np.ndarray:
        q_lens = np.diff(self.cu_q_lens)
        starts = np.concatenate([[0], np.cumsum(self.seq_lens)[:-1]])
        return np.concatenate([np.arange(s + L - n, s + L) for s, L, n in
                               zip(starts, self.seq_lens, q_lens)]).astype(np.int64)

    def cached_token_rows(self) -> np.ndarray:
        new = np.zeros(len(self.k), bool)
        new[self.new_token_rows()] = True
        return np.nonzero(~new)[0]


def make_prefill_case(seed: int, ctx_lens, new_lens, num_q_heads: int,
                      num_kv_heads: int, head_dim: int, table: str = "identity",
                      std: float = 1.0, window: int = 0, extra_pages: int = 0,
                      planted_below: int = 0, name: str = "prefill") -> PrefillCase:
    """planted_below > 0: a planted key at a seeded position below planted_below (and
    below every sequence's context), in every KV head g of every sequence, equal to
    8 * q / |q| for q the query of head g * G at the sequence's LAST new row."""
    rng = np.random.default_rng(seed)
    ctx_lens = np.asarray(ctx_lens, np.int64)
    new_lens = np.asarray(new_lens, np.int64)
    seq_lens = (ctx_lens + new_lens).astype(np.int32)
    B = len(seq_lens)
    Nq = int(new_lens.sum())
    T = int(seq_lens.sum())
    q = normal_bf16(rng, (Nq, num_q_heads, head_dim))
    k = normal_bf16(rng, (T, num_kv_heads, head_dim), std)
    v = normal_bf16(rng, (T, num_kv_heads, head_dim), std)
    meta = {}
    if planted_below > 0:
        G = num_q_heads // num_kv_heads
        pos = int(rng.integers(0, min(planted_below, int(ctx_lens.min()))))
        meta["planted_pos"] = pos
        starts = np.concatenate([[0], np.cumsum(seq_lens)[:-1]])
        ends = np.cumsum(new_lens) - 1
        for b in range(B):
            for g in range(num_kv_heads):
                qv = q[ends[b], g * G].astype(np.float64)
                k[starts[b] + pos, g] = bf16_round(
                    (8.0 * qv / np.linalg.norm(qv)).astype(np.float32))
    pages_per_seq = max(1, -(-int(seq_lens.max()) // PAGE_SIZE))
    num_pages = B * pages_per_seq + extra_pages
    bt = make_block_table(rng, B, pages_per_seq, table, num_pages)
    ts, tp, slots = token_layout(seq_lens, bt)
    cu = np.concatenate([[0], np.cumsum(new_lens)]).astype(np.int32)
    return PrefillCase(name, q, cu, k, v, ts, tp, slots, bt, seq_lens, num_pages,
                       num_kv_heads, head_dim, window, meta)


@dataclass
class LogitsCase:
    """Inputs of one paged-logits call: query rows q [R][Hq][D] grouped by request
    (cu_rows [B+1]), each row seeing the first row_lens[r] keys of its request's cache;
    k, v, token_* and slots cover every cached token as in DecodeCase."""
    name: str
    q: np.ndarray
    cu_rows: np.ndarray
    row_lens: np.ndarray
    k: np.ndarray
    v: np.ndarray
    token_seq: np.ndarray
    token_pos: np.ndarray
    slots: np.ndarray
    block_table: np.ndarray
    seq_lens: np.ndarray
    num_pages: int
    num_kv_heads: int
    head_dim: int


def make_logits_case(seed: int, seq_lens, rows_per_req, num_q_heads: int,
                     num_kv_heads: int, head_dim: int, table: str = "perm",
                     causal_rows: bool = True, std: float = 1.0, extra_pages: int = 0,
                     name: str = "logits") -> LogitsCase:
    """Requests with seq_lens cached tokens and rows_per_req query rows each; with
    causal_rows row i of request b sees seq_lens[b] - rows_per_req[b] + i + 1 keys (the
    rows are the request's last tokens), else every row sees the whole cache."""
    rng = np.random.default_rng(seed)
    seq_lens = np.asarray(seq_lens, np.int32)
    rows = np.asarray(rows_per_req, np.int64)
    B = len(seq_lens)
    R = int(rows.sum())
    T = int(seq_lens.sum())
    q = normal_bf16(rng, (R, num_q_heads, head_dim))
    k = normal_bf16(rng, (T, num_kv_heads, head_dim), std)
    v = normal_bf16(rng, (T, num_kv_heads, head_dim), std)
    lens = []
    for b in range(B):
        for i in range(int(rows[b])):
            L = int(seq_lens[b])
            lens.append(max(0, L - int(rows[b]) + i + 1) if causal_rows else L)
    pages_per_seq = max(1, -(-int(seq_lens.max()) // PAGE_SIZE)) if B else 1
    num_pages = B * pages_per_seq + extra_pages
    bt = make_block_table(rng, B, pages_per_seq, table, num_pages)
    ts, tp, slots = token_layout(seq_lens, bt)
    cu = np.concatenate([[0], np.cumsum(rows)]).astype(np.int32)
    return LogitsCase(name, q, cu, np.asarray(lens, np.int32), k, v, ts, tp, slots, bt,
                      seq_lens, num_pages, num_kv_heads, head_dim)


# --------------------------------------------------------------------------------
# The five named workloads.
# --------------------------------------------------------------------------------

def tiny_decode(seed: int = 101) -> DecodeCase:
    """1 sequence of 256 tokens, 4 query heads / 1 KV head, head_dim 64, identity
    table (16 pages), one decode query; N(0,1) bf16."""
    return make_decode_case(seed, [256], 4, 1, 64, table="identity", name="tiny_decode")


def llama8b_decode(seed: int = 102, seq_len: int = 20000, batch: int = 8) -> DecodeCase:
    """Llama-3.1-8B-shaped decode layer: 8 x 20,000 tokens, 32 q / 8 KV heads,
    head_dim 128, page size 16, block table a seeded permutation of all pages;
    K/V N(0,1) with 4 outlier channels per KV head scaled x20."""
    return make_decode_case(seed, [seq_len] * batch, 32, 8, 128, table="perm",
                            outliers=4, name="llama8b_decode")


def long_context_decode(seed: int = 103, seq_len: int = 131072) -> DecodeCase:
    """131,072-token accumulation stress: 32 q / 8 KV heads, head_dim 128, K/V
    N(0, 0.5) bf16 with a planted dominant key; identity table."""
    return make_decode_case(seed, [seq_len], 32, 8, 128, table="identity", std=0.5,
                            planted=True, name="long_context_decode")


def gptoss_hybrid_layer(layer: int, seed: int = 104, seq_len: int = 20000,
                        batch: int = 8) -> DecodeCase:
    """One layer of the gpt-oss-20b-shaped hybrid stack: 64 q / 8 KV heads,
    head_dim 64, 8 x 20,000 tokens, identity table shared by all layers; even
    layers full attention, odd layers sliding window 128."""
    window = 0 if layer % 2 == 0 else 128
    return make_decode_case(seed * 1000 + layer, [seq_len] * batch, 64, 8, 64,
                            table="identity", window=window,
                            name=f"gptoss_layer{layer}")


GPTOSS_LAYERS = 24


def hd256_prefill(seed: int = 105, ctx: int = 32768, new: int = 8192) -> PrefillCase:
    """head_dim-256 chunked prefill: 8,192 new queries appended to a 32,768-token
    cache, 8 q / 4 KV heads, causal, identity table, N(0,1) bf16."""
    return make_prefill_case(seed, [ctx], [new], 8, 4, 256, table="identity",
                             name="hd256_prefill")


def long_context_prefill(seed: int = 106, ctx: int = 130944, new: int = 128) -> PrefillCase:
    """Accumulation stress for the FP8-MFMA prefill: 128 new queries at the end of a
    131,072-token sequence, 32 q / 8 KV heads, head_dim 128, K/V N(0, 0.5) bf16 with a
    planted key 8 q / |q| (q of the last new row, first head of each group) at a seeded
    position in the first 16,384 tokens, so that nearly every key is read after it."""
    return make_prefill_case(seed, [ctx], [new], 32, 8, 128, table="identity", std=0.5,
                             planted_below=16384, name="long_context_prefill")
