"""CPU oracle for FP8 (e4m3) paged KV-cache attention.  TEST INFRASTRUCTURE ONLY.

A plain, slow, obviously correct float64/numpy statement of what the device path
computes, written from the pages' description of vLLM's FP8 KV cache:
  e4m3.py       code table and round-to-nearest-even saturating encoder
  cache.py      per-tensor / per-token-head scales, quantisation, paged cache write,
                query quantisation
  attention.py  float64 softmax attention (decode and chunked prefill) through a
                block table, GQA, sliding window
  scales.py     host scale resolution (sentinels, single kv scale) and the
                sliding-window skip policy
  logits.py     float64 paged query-key logits per query head (a sparse-attention
                indexer's scores), through a block table, GQA, per-row visibility

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this package.  It shares no code with the device path
(``fp8_quantized_paged_amd``), and neither imports the other; the only common code
is the seeded input generator package ``workloads``, which holds none of the
method's arithmetic.

Pins (tests/test_oracle_*.py): the decode table against the format's printed facts
and torch's float8_e4m3fn view of all 256 codes; the encoder by round trip over
every finite code, an exhaustive sweep over all 65,536 bf16 patterns at several
scales against torch's saturating cast, and every midpoint between neighbouring
codes; scales by closed form and invariants; attention by equal keys, a dominant
key, lossless grid values, GQA grouping, windows, page permutation, prefill/decode
agreement and a brute-force pure-Python softmax; logits by pure-Python dot products
over slot-addressed rows, one-hot queries (a lookup), constant key heads (GQA closed
form), visibility counts, page permutation and bilinearity.

Parity unpinned: nothing in this package.  (The effect of quantising softmax
probabilities to e4m3 inside the device's prefill kernel is not emulated here -- it
depends on the kernel's tiling; attention.attend_rows instead bounds the move of the
renormalised output under given per-key relative weight errors, pinned by brute force
over every corner of the error box, and the tests compare the device result with the
exact attention within that bound.)
"""
