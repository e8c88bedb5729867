"""Benchmark: FP8 paged decode attention on the Llama-3.1-8B-shaped decode layer.

Workload (one "step" = the whole decode hot path for one batch): 8 sequences of
20,000 tokens, 32 query / 8 KV heads, head_dim 128, page size 16, block table a
seeded permutation of all 10,000 pages, K/V bf16 N(0,1) with 4 outlier channels per
KV head scaled x20, fp8 e4m3 cache with per-token-head scales.  Each step writes
the 8 current tokens through the quantising cache write, then runs the split-K
decode (fused query quantisation and split merge) over all 20,000 keys of every
sequence.  Inputs are resident in HBM before timing starts; steps rotate over four
independent cache copies (4 x 338 MB) so the 256 MB Infinity Cache cannot serve a
step from the previous one.

Prints ONE JSON line.  `value` = algorithmic bytes of the step / measured step time
(GB/s).  `roofline` covers the decode kernel alone (HIP events around each decode
launch, on the stream it runs on).  `cpu_baseline` times the CPU oracle (float64)
on a bounded sample of the same step (a subset of the sequences).
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0      # MI355X HBM3E, AMD published
METRIC = "fp8 paged decode attention: HBM GB/s (% of peak), µs/step at 8×20k ctx"
PROFILE_TRAFFIC = os.path.join(ROOT, "profiles", "decode_llama8b_traffic.json")


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--rotate", type=int, default=4, help="independent cache copies")
    ap.add_argument("--cpu-seqs", type=int, default=8,
                    help="sequences in the oracle's timed sample (0 = skip)")
    ap.add_argument("--cpu-reps", type=int, default=2,
                    help="repetitions of the oracle's timed sample")
    ap.add_argument("--no-bf16", action="store_true", help="skip the bf16-cache leg")
    ap.add_argument("--copy-calib", action="store_true",
                    help="also run a plain 1 GiB device copy (counter calibration)")
    return ap.parse_args()


def step_bytes(B, L, Hkv, Hq, D, scale_bytes):
    """Algorithmic bytes.  decode: per (token, KV head) D K codes + D V codes + K/V
    scales; plus q and out (bf16) and the block table.  write: per new (token, head)
    read 2D bf16 values x2 (K, V), write D codes x2 and the scales."""
    pages = (L + 15) // 16
    dec = B * L * Hkv * (2 * D + scale_bytes) + 2 * (B * Hq * D * 2) + B * pages * 4
    wr = B * Hkv * (2 * 2 * D + 2 * D + scale_bytes)
    return dec, wr


def kernel_source_hash() -> str:
    h = hashlib.sha256()
    for f in ("decode.hip", "kvq_device.h"):
        h.update(open(os.path.join(ROOT, "fp8_quantized_paged_amd", "csrc", f), "rb").read())
    return h.hexdigest()[:16]


def measured_traffic():
    """HBM bytes per decode launch from the committed counter profile, if it was
    taken on the current kernel source; else None."""
    try:
        prof = json.load(open(PROFILE_TRAFFIC))
    except (OSError, ValueError):
        return None
    if prof.get("kernel_source_hash") != kernel_source_hash():
        return None
    return prof.get("bytes_per_launch")


def cpu_baseline(case, nseq, reps=1):
    """Time the oracle on the step restricted to ``nseq`` sequences: quantise the new
    token's K/V into the oracle's cache, quantise q, read (dequantise) the cache and
    run float64 attention.  Building the rest of the cache is setup, not timed."""
    import numpy as np
    from oracle import attention, cache as ocache

    B = len(case.seq_lens)
    L = int(case.seq_lens[0])
    P = (L + 15) // 16
    Hkv, D = case.num_kv_heads, case.head_dim
    work = []
    for b in range(nseq):
        rows = np.nonzero(case.token_seq == b)[0]
        pages = case.block_table[b]
        local = {int(p): i for i, p in enumerate(pages)}       # compact page pool
        bt = np.arange(P, dtype=np.int32)[None]
        slots = np.array([local[int(s) // 16] * 16 + int(s) % 16 for s in case.slots[rows]])
        pools = ocache.new_pools(P, Hkv, D)
        ocache.cache_write(pools, case.k[rows[:-1]], case.v[rows[:-1]], slots[:-1],
                           "per_token_head")
        work.append((b, rows, bt, slots, pools))
    t0 = time.perf_counter()
    for _ in range(reps):
        for b, rows, bt, slots, pools in work:
            ocache.cache_write(pools, case.k[rows[-1:]], case.v[rows[-1:]], slots[-1:],
                               "per_token_head")
            _, qh = ocache.quantize_q(case.q[b:b + 1], 1.0)
            attention.decode(qh, ocache.dequantized(pools, "k"),
                             ocache.dequantized(pools, "v"), bt, np.array([L]))
    dt = (time.perf_counter() - t0) / reps
    dec, wr = step_bytes(nseq, L, Hkv, case.num_q_heads, D, 8)
    try:
        from threadpoolctl import threadpool_info
        blas = max((i.get("num_threads", 1) for i in threadpool_info()), default=1)
    except Exception:  # pragma: no cover
        blas = None
    cores = len(os.sched_getaffinity(0))
    return {"value": (dec + wr) / dt / 1e9, "unit": "GB/s", "cores": cores,
            "kind": "oracle", "seconds": dt, "blas_threads": blas,
            "sample": f"{nseq} of {B} sequences of one decode step (same inputs: new-token "
                      f"cache write, q quantisation, cache read, float64 attention), mean "
                      f"of {reps} runs; value = their algorithmic bytes / oracle seconds"}


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}); this build "
              "has no multi-GPU path", file=sys.stderr)
        sys.exit(2)
    import numpy as np
    import torch

    import fp8_quantized_paged_amd as kvq
    import workloads

    def log(*a):
        print(*a, file=sys.stderr, flush=True)

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    case = workloads.llama8b_decode()
    B, Hq, D = case.q.shape
    Hkv = case.num_kv_heads
    L = int(case.seq_lens[0])
    log(f"bench: workload generated (B={B} L={L} Hq={Hq} Hkv={Hkv} D={D})")

    def to_dev(x):
        bits = workloads.bf16_bits(x).view(np.int16)
        return torch.from_numpy(np.ascontiguousarray(bits)).view(torch.bfloat16).to(dev)

    last = case.last_token_rows()
    hist = np.setdiff1d(np.arange(len(case.k)), last)
    q = to_dev(case.q)
    k_new, v_new = to_dev(case.k[last]), to_dev(case.v[last])
    slots_new = torch.from_numpy(case.slots[last].astype(np.int64)).to(dev)
    bt = torch.from_numpy(case.block_table).to(dev)
    sl = torch.from_numpy(case.seq_lens).to(dev)
    scales = kvq.Scales(1.0, 1.0, 1.0, 1.0)

    def build_caches(dtype, n):
        caches = [kvq.PagedCache(case.num_pages, Hkv, D, dtype, "per_token_head")
                  for _ in range(n)]
        step = 16384
        for i in range(0, len(hist), step):
            sel = hist[i:i + step]
            kk, vv = to_dev(case.k[sel]), to_dev(case.v[sel])
            ss = torch.from_numpy(case.slots[sel].astype(np.int64)).to(dev)
            for c in caches:
                kvq.cache_write(c, kk, vv, ss)
        torch.cuda.synchronize()
        return caches

    def run(caches, steps, warmup, events=True):
        ws = kvq.decode_workspace(caches[0], B, Hq, L, 0, 0, dev)
        out = torch.empty((B, Hq, D), dtype=torch.bfloat16, device=dev)
        for i in range(warmup):
            c = caches[i % len(caches)]
            kvq.cache_write(c, k_new, v_new, slots_new)
            kvq.decode_attention(c, q, bt, sl, L, scales, out=out, workspace=ws)
        torch.cuda.synchronize()
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
              for _ in range(steps)] if events else []
        t0 = torch.cuda.Event(enable_timing=True)
        t1 = torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        t0.record()
        for i in range(steps):
            c = caches[i % len(caches)]
            kvq.cache_write(c, k_new, v_new, slots_new)
            if events:
                ev[i][0].record()
            kvq.decode_attention(c, q, bt, sl, L, scales, out=out, workspace=ws)
            if events:
                ev[i][1].record()
        t1.record()
        torch.cuda.synchronize()
        step_ms = t0.elapsed_time(t1) / steps
        dec_ms = [a.elapsed_time(b) for a, b in ev]
        return step_ms, dec_ms

    fp8_caches = build_caches("fp8", args.rotate)
    log("bench: fp8 caches filled")
    step_ms, dec_ms = run(fp8_caches, args.steps, args.warmup)
    dec_bytes, wr_bytes = step_bytes(B, L, Hkv, Hq, D, 8)
    dec_us = float(np.mean(dec_ms)) * 1e3
    achieved = dec_bytes / (dec_us * 1e-6) / 1e9
    result = {
        "metric": METRIC,
        "value": round((dec_bytes + wr_bytes) / (step_ms * 1e-3) / 1e9, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(step_ms, 5),
        "us_per_step": round(step_ms * 1e3, 2),
        "pct_hbm_peak": round(100 * (dec_bytes + wr_bytes) / (step_ms * 1e-3) / 1e9
                              / HBM_PEAK_GBS, 2),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp8_e4m3",
        "data": "synthetic",
        "config": {"workload": "Llama-3.1-8B-shaped decode layer: 8 seqs x 20,000 ctx, "
                               "32 q / 8 KV heads, head_dim 128, page 16, permuted block "
                               "table, fp8 e4m3 cache with per-token-head scales; step = "
                               "cache write of 8 new tokens + split-K decode",
                   "batch": B, "context": L, "q_heads": Hq, "kv_heads": Hkv,
                   "head_dim": D, "page_size": 16, "scale_mode": "per_token_head",
                   "accumulate": "f32", "cache_copies_rotated": args.rotate,
                   "step_bytes": dec_bytes + wr_bytes, "decode_bytes": dec_bytes},
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": measured_traffic(), "kernel": "decode_split_kernel",
                     "kernel_us": round(dec_us, 2),
                     "kernel_us_p10_p90": [round(float(np.percentile(dec_ms, 10)) * 1e3, 2),
                                           round(float(np.percentile(dec_ms, 90)) * 1e3, 2)]},
    }
    del fp8_caches
    torch.cuda.empty_cache()
    if not args.no_bf16:
        bf_caches = build_caches("bf16", 2)
        bf_ms, bf_dec = run(bf_caches, max(10, args.steps // 2), args.warmup)
        pages = (L + 15) // 16
        bdec = B * L * Hkv * 4 * D + 2 * (B * Hq * D * 2) + B * pages * 4  # bf16 K+V
        result["bf16_cache_baseline"] = {
            "us_per_step": round(bf_ms * 1e3, 2),
            "decode_us": round(float(np.mean(bf_dec)) * 1e3, 2),
            "GB_s": round(bdec / (float(np.mean(bf_dec)) * 1e-3) / 1e9, 1),
            "fp8_over_bf16_step_time": round(step_ms / bf_ms, 3)}
        del bf_caches
        torch.cuda.empty_cache()
    if args.copy_calib:
        n = 1 << 30
        src = torch.empty(n, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        result["copy_calib_bytes"] = n
    if args.cpu_seqs > 0:
        log("bench: timing the CPU oracle sample")
        result["cpu_baseline"] = cpu_baseline(case, min(args.cpu_seqs, B), args.cpu_reps)
    else:
        result["cpu_baseline"] = None
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
