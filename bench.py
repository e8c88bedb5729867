"""Benchmark: FP8 paged attention hot path on one MI355X.

Headline (the JSON line's `value`): the Llama-3.1-8B-shaped decode layer — 8
sequences of 20,000 tokens, 32 query / 8 KV heads, head_dim 128, page size 16, block
table a seeded permutation of all 10,000 pages, K/V bf16 N(0,1) with 4 outlier
channels per KV head scaled x20, fp8 e4m3 cache with per-token-head scales.  One step
is one launch of the fused decode step: it stores the 8 current tokens (quantised as
the cache write does) and runs the split-K decode (fused query quantisation and split
merge) over all 20,000 keys of every sequence.  The same step as two launches (cache
write, then decode) is timed beside it.  Inputs are resident in HBM before timing
starts; steps rotate over four independent cache copies (4 x 338 MB) so the 256 MB
Infinity Cache cannot serve a step from the previous one.  `value` = algorithmic bytes of the step / step time (GB/s).

`roofline` covers the decode kernel alone (HIP events around a burst of back-to-back
fused launches, on the stream they run on).  Further legs, each timed the same way, are
reported beside it: the bf16-cache baseline of the same layer, the tiny decode, the 131,072-token decode,
the 24-layer gpt-oss-20b-shaped hybrid step (12 fp8 full layers + 12 bf16 window-128
layers, cache writes included), the head_dim-256 chunked prefill (FP8 matrix cores,
`roofline` against the dense FP8 peak, and its level-2 accumulation ablation), the bulk
quantising cache write (GB/s), and a compact inter-token-latency sweep (decode step of
whole models at 4k / 32k / 128k contexts, fp8 vs bf16 vs the bf16 window-layer skip
path: slopes, slope ratios, break-even contexts).  `cpu_baseline` times the CPU oracle
(float64) on the headline step's inputs.
"""
from __future__ import annotations

import argparse
import glob
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0        # MI355X HBM3E, AMD published
FP8_PEAK_TFLOPS = 5000.0     # MI355X dense FP8 matrix throughput, AMD published
METRIC = "fp8 paged decode attention: HBM GB/s (% of peak), µs/step at 8×20k ctx"
PROFILE_TRAFFIC = os.path.join(ROOT, "profiles", "decode_llama8b_traffic.json")
DECODE_KERNEL = "decode_kernel"
COPY_BYTES = 1 << 30
SETTLE_S = 0.1               # untimed steps after the warmup, before each timed region
LEGS = ("decode", "bf16", "tiny", "long", "hybrid", "prefill", "cache_write", "itl")
ITL_CONTEXTS = (4096, 32768, 131072)   # the default line's compact sweep
EXTRA_LEGS = ("prefill_d128", "prefill_d64", "per_kv_head", "prefill_bf16_window",
              "paged_logits", "prefill_split")
BF16_PEAK_TFLOPS = 2500.0    # MI355X dense bf16 matrix throughput, AMD published


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--rotate", type=int, default=4, help="independent cache copies")
    ap.add_argument("--legs", default=",".join(LEGS),
                    help=f"comma-separated subset of {LEGS}; 'decode' is the headline")
    ap.add_argument("--cpu-seqs", type=int, default=8,
                    help="sequences in the oracle's timed sample (0 = skip)")
    ap.add_argument("--cpu-reps", type=int, default=8,
                    help="repetitions of the oracle's timed sample (about 1.4 s each on "
                         "16 host cores: the default is ~11 s of CPU work)")
    ap.add_argument("--copy-calib", action="store_true",
                    help=f"also run a plain {COPY_BYTES >> 20} MiB device copy (counter "
                         "calibration for the HBM traffic figures)")
    ap.add_argument("--traffic-from", default="",
                    help="FETCH_SIZE,WRITE_SIZE rocprofv3 --pmc output directories (csv): "
                         "write the decode kernel's measured HBM bytes per launch to "
                         "profiles/ and exit (no GPU needed)")
    ap.add_argument("--itl", action="store_true",
                    help="instead of the headline: the attention-only inter-token-latency "
                         "sweep over context lengths (fp8 vs bf16 vs bf16 sliding-window "
                         "layers) and its slopes; prints its own JSON line")
    ap.add_argument("--itl-contexts", default="1024,4096,16384,32768,65536,131072",
                    help="context lengths of the --itl sweep")
    return ap.parse_args()


def log(*a):
    print(*a, file=sys.stderr, flush=True)


# ---- algorithmic work -------------------------------------------------------------------

def decode_bytes(B, L, Hkv, Hq, D, elem, scale_bytes, window=0):
    """Bytes a decode launch must move: per visible (token, KV head) 2D code bytes (or
    4D for bf16) and the per-token scales, plus q and out (bf16) and the block-table
    entries of the visible pages."""
    vis = min(L, window) if window > 0 else L
    pages = (vis + 15) // 16 + (1 if window > 0 else 0)
    return (B * vis * Hkv * (2 * D * elem + scale_bytes) + 2 * (B * Hq * D * 2)
            + B * min(pages, (L + 15) // 16) * 4)


def write_bytes(T, Hkv, D, elem, scale_bytes):
    """Cache write of T new tokens: read K and V (bf16), write the codes and scales."""
    return T * Hkv * (2 * 2 * D + 2 * D * elem + scale_bytes)


def prefill_flops(ctx, new, Hq, D):
    """4 D flops (QK^T and PV multiply-adds) per (query row, visible key, query head)."""
    return 4.0 * D * Hq * sum(ctx + i + 1 for i in range(new))


# ---- measured traffic (rocprofv3 --pmc) ---------------------------------------------------

def kernel_source_hash() -> str:
    h = hashlib.sha256()
    for f in ("decode.hip", "kvq_device.h"):
        h.update(open(os.path.join(ROOT, "fp8_quantized_paged_amd", "csrc", f), "rb").read())
    return h.hexdigest()[:16]


def measured_traffic():
    """HBM bytes per decode launch from the committed counter profile, if it was taken
    on the current kernel source; else None."""
    try:
        prof = json.load(open(PROFILE_TRAFFIC))
    except (OSError, ValueError):
        return None
    if prof.get("kernel_source_hash") != kernel_source_hash():
        return None
    return prof.get("bytes_per_launch")


def _counter_rows(directory):
    import csv
    rows = []
    for path in glob.glob(os.path.join(directory, "**", "*counter_collection.csv"),
                          recursive=True):
        with open(path) as f:
            rows.extend(csv.DictReader(f))
    if not rows:
        raise SystemExit(f"no *counter_collection.csv under {directory}")
    return rows


def _per_dispatch(rows, counter, name_part):
    vals = {}
    for r in rows:
        if r.get("Counter_Name") != counter or name_part not in r.get("Kernel_Name", ""):
            continue
        key = r.get("Dispatch_Id") or r.get("Correlation_Id")
        vals[key] = vals.get(key, 0.0) + float(r["Counter_Value"])
    return list(vals.values())


def write_traffic_profile(fetch_dir, write_dir):
    """FETCH_SIZE and WRITE_SIZE (KiB per dispatch) of the decode kernel, scaled by what
    the same counters read for the plain 1 GiB device copy (the runtime's copy kernel),
    averaged over dispatches."""
    import statistics
    fr, wr = _counter_rows(fetch_dir), _counter_rows(write_dir)
    dec_f = _per_dispatch(fr, "FETCH_SIZE", DECODE_KERNEL)
    dec_w = _per_dispatch(wr, "WRITE_SIZE", DECODE_KERNEL)
    # the calibration copy is the largest copy dispatch (others are small staging copies)
    cp_f = _per_dispatch(fr, "FETCH_SIZE", "copy")
    cp_w = _per_dispatch(wr, "WRITE_SIZE", "copy")
    if not (dec_f and dec_w and cp_f and cp_w):
        raise SystemExit("decode or copy dispatches missing in the counter files")
    f_scale = COPY_BYTES / (max(cp_f) * 1024.0)
    w_scale = COPY_BYTES / (max(cp_w) * 1024.0)
    fetch = statistics.mean(dec_f) * 1024.0 * f_scale
    write = statistics.mean(dec_w) * 1024.0 * w_scale
    prof = {"kernel": DECODE_KERNEL, "kernel_source_hash": kernel_source_hash(),
            "fetch_bytes_per_launch": round(fetch), "write_bytes_per_launch": round(write),
            "bytes_per_launch": round(fetch + write),
            "fetch_scale_from_copy": f_scale, "write_scale_from_copy": w_scale,
            "dispatches": [len(dec_f), len(dec_w)]}
    with open(PROFILE_TRAFFIC, "w") as f:
        json.dump(prof, f, indent=1)
    print(json.dumps(prof))


# ---- CPU baseline -------------------------------------------------------------------------

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
    dec = decode_bytes(nseq, L, Hkv, case.num_q_heads, D, 1, 8)
    wr = write_bytes(nseq, Hkv, D, 1, 8)
    try:
        from threadpoolctl import threadpool_info
        blas = max((i.get("num_threads", 1) for i in threadpool_info()), default=1)
    except Exception:  # pragma: no cover
        blas = None
    cores = len(os.sched_getaffinity(0))
    return {"value": round((dec + wr) / dt / 1e9, 4), "unit": "GB/s", "cores": cores,
            "kind": "oracle", "seconds": round(dt, 4), "blas_threads": blas,
            "sample": f"{nseq} of {B} sequences of one decode step (same inputs: new-token "
                      f"cache write, q quantisation, cache read, float64 attention), mean "
                      f"of {reps} runs ({dt * reps:.1f} s of CPU work in all); value = their "
                      f"algorithmic bytes / oracle seconds per run"}


# ---- attention-only inter-token latency over context length ---------------------------------

def run_itl(args):
    """--itl: the sweep at --itl-contexts, printed as its own JSON line."""
    res = itl_sweep([int(x) for x in args.itl_contexts.split(",") if x])
    print(json.dumps(res), flush=True)


def itl_sweep(contexts):
    """Per decode step, the attention of every layer of a model (fused new-token write +
    decode, one HIP graph replay per step), over context lengths: Llama-3.1-8B-shaped
    (32 layers, 8 sequences, 32/8 heads, D 128) with an fp8 (per-token-head) or a bf16
    cache, and gpt-oss-20b-shaped (24 layers alternating full attention and a 128-token
    window, 8 sequences, 64/8 heads, D 64) with every layer fp8, every layer bf16, or
    full layers fp8 and window layers bf16 (the skip path).  Step time = a + slope *
    context is fitted per variant; the fp8 / bf16 slope ratio and the context where fp8
    overtakes bf16 follow.  Layers rotate over distinct caches totalling >= 1 GiB (>
    the 256 MB Infinity Cache), so no layer is served from the previous one; window
    layers keep only their visible pages (the rest of their block table points at a
    page they never read)."""
    import numpy as np
    import torch

    import fp8_quantized_paged_amd as kvq

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    ones = kvq.Scales(1.0, 1.0, 1.0, 1.0)
    gen = torch.Generator(device=dev)
    gen.manual_seed(20240607)

    def make_layer(B, L, Hq, Hkv, D, dtype, window):
        """One layer's cache holding L tokens per sequence (N(0,1) bf16 rows through the
        cache write), its block table, query and new-token rows."""
        pages = (L + 15) // 16
        if window:
            vis = (window + 15) // 16 + 1
            first = max(0, pages - vis)
            P = B * (pages - first) + 1
            bt = torch.zeros((B, pages), dtype=torch.int32, device=dev)
            own = torch.arange(1, P, dtype=torch.int32, device=dev).reshape(B, -1)
            bt[:, first:] = own
        else:
            first = 0
            P = B * pages
            bt = torch.arange(P, dtype=torch.int32, device=dev).reshape(B, pages)
        c = kvq.PagedCache(P, Hkv, D, dtype, "per_token_head")
        # slots of every written token (positions first*16 .. L-1 of each sequence)
        pos = torch.arange(first * 16, L, device=dev)
        slots = (bt[:, (pos // 16)].to(torch.int64) * 16 + pos % 16).reshape(-1)
        for i in range(0, slots.numel(), 1 << 18):
            sl = slots[i:i + (1 << 18)]
            k = torch.randn((sl.numel(), Hkv, D), device=dev, generator=gen).to(torch.bfloat16)
            v = torch.randn((sl.numel(), Hkv, D), device=dev, generator=gen).to(torch.bfloat16)
            kvq.cache_write(c, k, v, sl)
        q = torch.randn((B, Hq, D), device=dev, generator=gen).to(torch.bfloat16)
        kn = torch.randn((B, Hkv, D), device=dev, generator=gen).to(torch.bfloat16)
        vn = torch.randn((B, Hkv, D), device=dev, generator=gen).to(torch.bfloat16)
        ws = kvq.decode_workspace(c, B, Hq, L, window, 0, dev)
        return (c, q, kn, vn, bt, torch.full((B,), L, dtype=torch.int32, device=dev),
                window, ws, c.nbytes)

    def step_us(layers, order, B, Hq, D, L):
        out = torch.empty((B, Hq, D), dtype=torch.bfloat16, device=dev)

        def step():
            for i in order:
                c, q, kn, vn, bt, sl, win, ws, _ = layers[i]
                kvq.decode_step(c, q, kn, vn, bt, sl, L, ones, window=win, out=out,
                                workspace=ws)
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            step()
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            step()
        for _ in range(3):
            g.replay()
        torch.cuda.synchronize()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        n = 10
        e0.record()
        for _ in range(n):
            g.replay()
        e1.record()
        torch.cuda.synchronize()
        del g
        return e0.elapsed_time(e1) * 1e3 / n

    def model_step(nlayers, kinds, B, Hq, Hkv, D, L):
        """kinds[i]: (dtype, window) of layer i; distinct caches per kind until >= 1 GiB."""
        layers, order, by_kind = [], [], {}
        for i in range(nlayers):
            kind = kinds[i % len(kinds)]
            lst = by_kind.setdefault(kind, [])
            total = sum(layers[j][-1] for j in lst)
            if len(lst) < 2 or (total < (1 << 30) and len(lst) < nlayers):
                layers.append(make_layer(B, L, Hq, Hkv, D, kind[0], kind[1]))
                lst.append(len(layers) - 1)
            order.append(lst[i // len(kinds) % len(lst)])
        us = step_us(layers, order, B, Hq, D, L)
        del layers
        torch.cuda.empty_cache()
        return us

    models = {
        "llama-3.1-8b (32 layers, 8 seqs, 32/8 heads, D 128)": (
            32, 8, 32, 8, 128,
            {"fp8": [("fp8", 0)], "bf16": [("bf16", 0)]}),
        "gpt-oss-20b (24 layers alternating full / window 128, 8 seqs, 64/8 heads, D 64)": (
            24, 8, 64, 8, 64,
            {"fp8": [("fp8", 0), ("fp8", 128)], "bf16": [("bf16", 0), ("bf16", 128)],
             "fp8 + bf16 window layers": [("fp8", 0), ("bf16", 128)]}),
    }
    res = {"metric": "attention-only decode step time vs context (inter-token latency "
                     "slope)", "unit": "us per step", "contexts": contexts, "models": {}}
    for mname, (nl, B, Hq, Hkv, D, variants) in models.items():
        mres = {}
        for vname, kinds in variants.items():
            times = []
            for L in contexts:
                t = model_step(nl, kinds, B, Hq, Hkv, D, L)
                times.append(round(t, 1))
                log(f"itl: {mname.split(' ')[0]} {vname} ctx {L}: {t:.1f} us")
            slope, icpt = np.polyfit(np.asarray(contexts, float), np.asarray(times), 1)
            mres[vname] = {"us": times, "slope_us_per_1k_ctx": round(slope * 1e3, 3),
                           "intercept_us": round(icpt, 1)}
        base = mres["bf16"]["slope_us_per_1k_ctx"]
        for vname, v in mres.items():
            if vname == "bf16":
                continue
            v["slope_ratio_vs_bf16"] = round(v["slope_us_per_1k_ctx"] / base, 3)
            ds = base - v["slope_us_per_1k_ctx"]
            di = v["intercept_us"] - mres["bf16"]["intercept_us"]
            v["break_even_ctx_vs_bf16"] = round(di / ds * 1e3) if ds > 0 and di > 0 else 0
        res["models"][mname] = mres
    return res


# ---- GPU legs -------------------------------------------------------------------------------

def mfma_ceiling(torch, dev):
    """Sustained rate of the prefill's FP8 matrix instruction (32x32x64, 131,072 flops per
    wave and instruction) from the measurement probe libkvq_probe.so: four independent
    accumulator chains per wave, 1, 2 and 4 waves per SIMD; the best rate is reported.
    None when the probe library was not built."""
    import ctypes
    path = os.path.join(ROOT, "fp8_quantized_paged_amd", "libkvq_probe.so")
    if not os.path.exists(path):
        return None
    lib = ctypes.CDLL(path)
    fn = lib.kvq_probe_mfma_rate
    fn.restype = ctypes.c_int
    fn.argtypes = [ctypes.c_int32, ctypes.c_int32, ctypes.c_void_p, ctypes.c_void_p]
    iters = 4000
    best = (0.0, 0)
    rates = {}
    for blocks in (256, 512, 1024):
        out = torch.empty(blocks * 256, dtype=torch.float32, device=dev)
        st = torch.cuda.current_stream().cuda_stream
        for _ in range(3):
            assert fn(blocks, iters, out.data_ptr(), st) == 0
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(5):
            assert fn(blocks, iters, out.data_ptr(), st) == 0
        e1.record()
        torch.cuda.synchronize()
        sec = e0.elapsed_time(e1) * 1e-3 / 5
        tfl = blocks * 4 * iters * 4 * 131072 / sec / 1e12
        rates[f"{blocks // 256}_waves_per_simd"] = round(tfl, 1)
        if tfl > best[0]:
            best = (tfl, blocks)
    return {"TFLOP_s": round(best[0], 1), "frac_of_published": round(best[0] / FP8_PEAK_TFLOPS, 4),
            "waves_per_simd": best[1] // 256, "by_waves_per_simd": rates,
            "probe": "back-to-back v_mfma_f32_32x32x64_f8f6f4, four independent chains per "
                     "wave, 256 workgroups of 4 waves per wave-per-SIMD step"}


class Timer:
    """HIP events on torch's current stream, which is the stream libkvq launches on."""

    def __init__(self, torch):
        self.torch = torch

    def run(self, fn, steps, warmup, warm_ms=0.0):
        """warm_ms: after the warm-up launches, keep launching until that much wall time
        has passed, so the leg is timed at the clock it settles at.  After the
        memory-bound legs the compute clock takes ~100 launches of a 1.5 ms kernel to come
        back up (head_dim-256 prefill: mean 1681 us after 3 warm-up launches, 1525 us
        after 100 or 300).  The headline decode step keeps its plain warm-up count."""
        torch = self.torch
        for i in range(warmup):
            fn(i)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        while (time.perf_counter() - t0) * 1e3 < warm_ms:
            for i in range(4):
                fn(i)
            torch.cuda.synchronize()
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
              for _ in range(steps)]
        for i in range(steps):
            ev[i][0].record()
            fn(i)
            ev[i][1].record()
        torch.cuda.synchronize()
        return [a.elapsed_time(b) * 1e3 for a, b in ev]  # µs


def stats(us):
    import numpy as np
    return {"us_mean": round(float(np.mean(us)), 2), "us_median": round(float(np.median(us)), 2),
            "us_p10_p90": [round(float(np.percentile(us, 10)), 2),
                           round(float(np.percentile(us, 90)), 2)]}


def main():
    args = parse()
    if args.traffic_from:
        fetch_dir, write_dir = args.traffic_from.split(",")
        write_traffic_profile(fetch_dir, write_dir)
        return
    if args.itl:
        if args.gpus != 1:
            sys.exit("bench.py runs on one GPU only")
        run_itl(args)
        return
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}); this build "
              "has no multi-GPU path", file=sys.stderr)
        sys.exit(2)
    legs = [x for x in args.legs.split(",") if x]
    for x in legs:
        if x not in LEGS + EXTRA_LEGS:
            sys.exit(f"unknown leg {x!r}; choose from {LEGS + EXTRA_LEGS}")
    import numpy as np
    import torch

    import fp8_quantized_paged_amd as kvq
    import workloads

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    timer = Timer(torch)

    def to_dev(x):
        bits = workloads.bf16_bits(x).view(np.int16)
        return torch.from_numpy(np.ascontiguousarray(bits)).view(torch.bfloat16).to(dev)

    ones = kvq.Scales(1.0, 1.0, 1.0, 1.0)
    result = {}

    # ---- headline: Llama-shaped decode layer --------------------------------------------
    case = workloads.llama8b_decode()
    B, Hq, D = case.q.shape
    Hkv = case.num_kv_heads
    L = int(case.seq_lens[0])
    log(f"bench: llama-shaped workload generated (B={B} L={L} Hq={Hq} Hkv={Hkv} D={D})")
    last = case.last_token_rows()
    hist = np.setdiff1d(np.arange(len(case.k)), last)
    q = to_dev(case.q)
    k_new, v_new = to_dev(case.k[last]), to_dev(case.v[last])
    slots_new = torch.from_numpy(case.slots[last].astype(np.int64)).to(dev)
    bt = torch.from_numpy(case.block_table).to(dev)
    sl = torch.from_numpy(case.seq_lens).to(dev)

    def build_caches(dtype, n, mode="per_token_head"):
        caches = [kvq.PagedCache(case.num_pages, Hkv, D, dtype, mode) for _ in range(n)]
        step = 16384
        for i in range(0, len(hist), step):
            sel = hist[i:i + step]
            kk, vv = to_dev(case.k[sel]), to_dev(case.v[sel])
            ss = torch.from_numpy(case.slots[sel].astype(np.int64)).to(dev)
            for c in caches:
                kvq.cache_write(c, kk, vv, ss)
        torch.cuda.synchronize()
        return caches

    def decode_step_legs(caches, steps, warmup):
        """Step times of the fused decode step (one launch: new-token cache write +
        decode) and of the two separate calls, and the decode kernel's duration."""
        ws = kvq.decode_workspace(caches[0], B, Hq, L, 0, 0, dev)
        out = torch.empty((B, Hq, D), dtype=torch.bfloat16, device=dev)

        def fused(i):
            kvq.decode_step(caches[i % len(caches)], q, k_new, v_new, bt, sl, L, ones,
                            out=out, workspace=ws)

        def unfused(i):
            c = caches[i % len(caches)]
            kvq.cache_write(c, k_new, v_new, slots_new)
            kvq.decode_attention(c, q, bt, sl, L, ones, out=out, workspace=ws)

        def timed(step):
            # warmup, then untimed steps for SETTLE_S more (the GPU leaves its idle
            # clocks over some milliseconds: the first ~10 ms of steps after the host-side
            # cache fill run ~15% slower), then exactly `steps` steps launched back to
            # back between two synchronisations: the wall clock over them is the step time
            for i in range(warmup):
                step(i)
            torch.cuda.synchronize()
            t_settle, i = time.perf_counter(), 0
            while time.perf_counter() - t_settle < SETTLE_S:
                step(i)
                i += 1
                if i % 50 == 0:
                    torch.cuda.synchronize()
            torch.cuda.synchronize()
            span0 = torch.cuda.Event(enable_timing=True)
            span1 = torch.cuda.Event(enable_timing=True)
            t0 = time.perf_counter()
            span0.record()
            for i in range(steps):
                step(warmup + i)
            span1.record()
            torch.cuda.synchronize()
            return ((time.perf_counter() - t0) * 1e6 / steps,
                    span0.elapsed_time(span1) * 1e3 / steps)

        fused_wall, fused_span = timed(fused)
        unfused_wall, unfused_span = timed(unfused)
        # the decode kernel's own duration: HIP events around a burst of back-to-back
        # fused launches (rotating the caches), so that no per-launch event gap counts
        k0 = torch.cuda.Event(enable_timing=True)
        k1 = torch.cuda.Event(enable_timing=True)
        k0.record()
        for i in range(steps):
            fused(i)
        k1.record()
        torch.cuda.synchronize()
        # warm: the same burst on one cache copy, which the 256 MB last-level cache
        # partly holds from one launch to the next (the cold figure above is the one used)
        w0 = torch.cuda.Event(enable_timing=True)
        w1 = torch.cuda.Event(enable_timing=True)
        for i in range(warmup):
            fused(0)
        w0.record()
        for i in range(steps):
            fused(0)
        w1.record()
        torch.cuda.synchronize()
        return {"wall_us": fused_wall, "span_us": fused_span,
                "kernel_us": k0.elapsed_time(k1) * 1e3 / steps,
                "warm_kernel_us": w0.elapsed_time(w1) * 1e3 / steps,
                "unfused_wall_us": unfused_wall, "unfused_span_us": unfused_span}

    if "decode" in legs:
        caches = build_caches("fp8", args.rotate)
        log("bench: fp8 caches filled")
        legs_t = decode_step_legs(caches, args.steps, args.warmup)
        step_us, span_us, dk_us = legs_t["wall_us"], legs_t["span_us"], legs_t["kernel_us"]
        del caches
        torch.cuda.empty_cache()
        # a second denominator: what a plain 1 GiB device-to-device copy streams here
        # (bytes read + written per second), and the same burst timed warm
        csrc = torch.empty(COPY_BYTES, dtype=torch.uint8, device=dev)
        cdst = torch.empty_like(csrc)
        for _ in range(3):
            cdst.copy_(csrc)
        c0 = torch.cuda.Event(enable_timing=True)
        c1 = torch.cuda.Event(enable_timing=True)
        c0.record()
        for _ in range(10):
            cdst.copy_(csrc)
        c1.record()
        torch.cuda.synchronize()
        copy_gbs = 2 * COPY_BYTES / (c0.elapsed_time(c1) * 1e-3 / 10) / 1e9
        del csrc, cdst
        torch.cuda.empty_cache()
        dec_b = decode_bytes(B, L, Hkv, Hq, D, 1, 8)
        wr_b = write_bytes(B, Hkv, D, 1, 8)
        # the fused kernel moves the decode's bytes and the new tokens' write
        achieved = (dec_b + wr_b) / (dk_us * 1e-6) / 1e9
        result.update({
            "metric": METRIC,
            "value": round((dec_b + wr_b) / (step_us * 1e-6) / 1e9, 2),
            "unit": "GB/s",
            "n_gpus": 1,
            "steps": args.steps,
            "warmup": args.warmup,
            "ms_per_step": round(step_us / 1e3, 5),
            "us_per_step": round(step_us, 2),
            "gpu_span_us_per_step": round(span_us, 2),
            "unfused_us_per_step": round(legs_t["unfused_wall_us"], 2),
            "pct_hbm_peak": round(100 * (dec_b + wr_b) / (step_us * 1e-6) / 1e9 / HBM_PEAK_GBS, 2),
            "higher_is_better": True,
            "scaling": "weak",
            "vs_baseline": None,
            "dtype": "fp8_e4m3",
            "data": "synthetic",
            "config": {"workload": "Llama-3.1-8B-shaped decode layer: 8 seqs x 20,000 ctx, "
                                   "32 q / 8 KV heads, head_dim 128, page 16, permuted block "
                                   "table, fp8 e4m3 cache with per-token-head scales; step = "
                                   "cache write of 8 new tokens + split-K decode, fused in "
                                   "one launch",
                       "batch": B, "context": L, "q_heads": Hq, "kv_heads": Hkv,
                       "head_dim": D, "page_size": 16, "scale_mode": "per_token_head",
                       "accumulate": "f32", "cache_copies_rotated": args.rotate,
                       "step_bytes": dec_b + wr_b, "decode_bytes": dec_b},
            "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS,
                         "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                         "traffic": measured_traffic(), "kernel": DECODE_KERNEL,
                         "kernel_us": round(dk_us, 2),
                         "kernel_timing": "HIP events around a burst of back-to-back "
                                          "fused decode-step launches after the timed "
                                          "steps; achieved counts decode + write bytes"},
            "ceilings": {
                "device_copy_GB_s": round(copy_gbs, 1),
                "decode_frac_of_device_copy": round(achieved / copy_gbs, 4),
                "warm_kernel_us": round(legs_t["warm_kernel_us"], 2),
                "warm_GB_s": round((dec_b + wr_b) / (legs_t["warm_kernel_us"] * 1e-6) / 1e9, 1),
                "note": "device copy: torch copy_ of 1 GiB, read + written bytes per second; "
                        "warm: the same burst on one cache copy (338 MB, partly held by the "
                        "256 MB last-level cache between launches)"},
        })

    if "bf16" in legs:
        caches = build_caches("bf16", 2)
        bl = decode_step_legs(caches, max(10, args.steps // 2), args.warmup)
        t_step, dec_us = bl["wall_us"], bl["kernel_us"]
        del caches
        torch.cuda.empty_cache()
        bdec = decode_bytes(B, L, Hkv, Hq, D, 2, 0)
        result["bf16_cache_baseline"] = {
            "us_per_step": round(t_step, 2),
            "decode_us": round(dec_us, 2),
            "GB_s": round(bdec / (dec_us * 1e-6) / 1e9, 1),
            "decode_bytes": bdec}
        if "us_per_step" in result:
            result["bf16_cache_baseline"]["fp8_over_bf16_step_time"] = round(
                result["us_per_step"] / t_step, 3)
    del case, q, k_new, v_new
    torch.cuda.empty_cache()

    if "tiny" in legs:
        tc = workloads.tiny_decode()
        c = kvq.PagedCache(tc.num_pages, tc.num_kv_heads, tc.head_dim, "fp8", "per_token_head")
        kvq.cache_write(c, to_dev(tc.k), to_dev(tc.v),
                        torch.from_numpy(tc.slots.astype(np.int64)).to(dev))
        tq, tbt, tsl = to_dev(tc.q), torch.from_numpy(tc.block_table).to(dev), \
            torch.from_numpy(tc.seq_lens).to(dev)
        ws = kvq.decode_workspace(c, 1, 4, 256, 0, 0, dev)
        out = torch.empty((1, 4, 64), dtype=torch.bfloat16, device=dev)
        us = timer.run(lambda i: kvq.decode_attention(c, tq, tbt, tsl, 256, ones, out=out,
                                                      workspace=ws), 50, 5, warm_ms=200.0)
        result["tiny_decode"] = {"workload": "1 seq x 256 tokens, 4/1 heads, D 64, "
                                             "per-token-head", **stats(us)}

    gen = torch.Generator(device=dev)

    def dev_normal(shape, std, seed):
        gen.manual_seed(seed)
        return (torch.randn(shape, generator=gen, device=dev) * std).to(torch.bfloat16)

    if "long" in legs:
        # 131,072-token decode, 32/8 heads, D 128, N(0, 0.5^2), per-tensor scale 1.0,
        # identity table; two cache copies (2 x 268 MB) rotate
        Lc, P = 131072, 131072 // 16
        caches = []
        for cpy in range(2):
            c = kvq.PagedCache(P, 8, 128, "fp8", "per_tensor")
            for t0 in range(0, Lc, 16384):
                kk = dev_normal((16384, 8, 128), 0.5, 1030 + t0)
                vv = dev_normal((16384, 8, 128), 0.5, 1031 + t0)
                kvq.cache_write(c, kk, vv, torch.arange(t0, t0 + 16384, device=dev))
            caches.append(c)
        lq = dev_normal((1, 32, 128), 1.0, 1039)
        lbt = torch.arange(P, dtype=torch.int32, device=dev).reshape(1, -1)
        lsl = torch.tensor([Lc], dtype=torch.int32, device=dev)
        ws = kvq.decode_workspace(caches[0], 1, 32, Lc, 0, 0, dev)
        out = torch.empty((1, 32, 128), dtype=torch.bfloat16, device=dev)
        us = timer.run(lambda i: kvq.decode_attention(caches[i % 2], lq, lbt, lsl, Lc, ones,
                                                      out=out, workspace=ws),
                       max(10, args.steps // 2), args.warmup, warm_ms=200.0)
        nb = decode_bytes(1, Lc, 8, 32, 128, 1, 0)
        result["long_context_decode"] = {
            "workload": "1 seq x 131,072 tokens, 32/8 heads, D 128, per-tensor scale",
            **stats(us), "bytes": nb,
            "GB_s": round(nb / (float(np.mean(us)) * 1e-6) / 1e9, 1),
            "frac_hbm": round(nb / (float(np.mean(us)) * 1e-6) / 1e9 / HBM_PEAK_GBS, 4)}
        del caches
        torch.cuda.empty_cache()

    if "hybrid" in legs:
        # 24 layers: even = full attention over an fp8 cache (per-tensor 1.0), odd =
        # window 128 over a bf16 cache; 8 x 20,000 tokens, 64/8 heads, D 64; a step
        # writes each layer's 8 new tokens and runs its decode (one fused launch a layer)
        Bh, Lh, Hqh, Hkvh, Dh, W = 8, 20000, 64, 8, 64, 128
        Ph = Bh * ((Lh + 15) // 16)
        hbt = torch.arange(Ph, dtype=torch.int32, device=dev).reshape(Bh, -1)
        hsl = torch.full((Bh,), Lh, dtype=torch.int32, device=dev)
        fill = torch.tensor([b * (Ph // Bh) * 16 + t for b in range(Bh) for t in range(Lh - 1)],
                            dtype=torch.int64, device=dev)
        layers = []
        for layer in range(24):
            full = layer % 2 == 0
            c = kvq.PagedCache(Ph, Hkvh, Dh, "fp8" if full else "bf16", "per_tensor")
            for t0 in range(0, fill.numel(), 32768):
                sel = fill[t0:t0 + 32768]
                kk = dev_normal((sel.numel(), Hkvh, Dh), 1.0, 2000 + 100 * layer + t0 // 32768)
                vv = dev_normal((sel.numel(), Hkvh, Dh), 1.0, 5000 + 100 * layer + t0 // 32768)
                kvq.cache_write(c, kk, vv, sel)
            kn = dev_normal((Bh, Hkvh, Dh), 1.0, 9000 + layer)
            vn = dev_normal((Bh, Hkvh, Dh), 1.0, 9100 + layer)
            qn = dev_normal((Bh, Hqh, Dh), 1.0, 9200 + layer)
            win = 0 if full else W
            ws = kvq.decode_workspace(c, Bh, Hqh, Lh, win, 0, dev)
            layers.append((c, kn, vn, qn, win, ws))
        torch.cuda.synchronize()
        out = torch.empty((Bh, Hqh, Dh), dtype=torch.bfloat16, device=dev)

        def hybrid_step(i):
            for c, kn, vn, qn, win, ws in layers:
                kvq.decode_step(c, qn, kn, vn, hbt, hsl, Lh, ones, window=win, out=out,
                                workspace=ws)
        nsteps, nwarm = max(10, args.steps // 4), max(2, args.warmup // 2)
        us_eager = timer.run(hybrid_step, nsteps, nwarm, warm_ms=200.0)
        # the same step captured once in a HIP graph and replayed, as a serving loop
        # would run it: the 24 launches then cost no host time each
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            hybrid_step(0)
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            hybrid_step(0)
        us = timer.run(lambda i: graph.replay(), nsteps, nwarm, warm_ms=200.0)
        nb = 12 * (decode_bytes(Bh, Lh, Hkvh, Hqh, Dh, 1, 0) + write_bytes(Bh, Hkvh, Dh, 1, 0)) \
            + 12 * (decode_bytes(Bh, Lh, Hkvh, Hqh, Dh, 2, 0, window=W)
                    + write_bytes(Bh, Hkvh, Dh, 2, 0))
        result["hybrid_stack_step"] = {
            "workload": "gpt-oss-20b-shaped 24-layer step: 12 fp8 full layers + 12 bf16 "
                        "window-128 layers, 8 x 20,000 ctx, 64/8 heads, D 64; cache writes "
                        "included (fused decode step per layer); one HIP graph replay per "
                        "step",
            **stats(us), "bytes": nb,
            "GB_s": round(nb / (float(np.mean(us)) * 1e-6) / 1e9, 1),
            "frac_hbm": round(nb / (float(np.mean(us)) * 1e-6) / 1e9 / HBM_PEAK_GBS, 4),
            "eager_launches": {**stats(us_eager)}}
        del graph
        del layers
        torch.cuda.empty_cache()

    if "prefill" in legs:
        pc = workloads.hd256_prefill()
        log("bench: hd256 prefill workload generated")
        c = kvq.PagedCache(pc.num_pages, pc.num_kv_heads, pc.head_dim, "fp8", "per_token_head")
        for t0 in range(0, len(pc.k), 16384):
            sl_ = slice(t0, t0 + 16384)
            kvq.cache_write(c, to_dev(pc.k[sl_]), to_dev(pc.v[sl_]),
                            torch.from_numpy(pc.slots[sl_].astype(np.int64)).to(dev))
        pq = to_dev(pc.q)
        pcu = torch.from_numpy(pc.cu_q_lens).to(dev)
        pbt = torch.from_numpy(pc.block_table).to(dev)
        psl = torch.from_numpy(pc.seq_lens).to(dev)
        n_new = int(pc.cu_q_lens[1])
        out = torch.empty(pc.q.shape, dtype=torch.bfloat16, device=dev)
        us = timer.run(lambda i: kvq.prefill_attention(c, pq, pcu, pbt, psl, n_new, ones,
                                                       out=out), 10, 3, warm_ms=200.0)
        fl = prefill_flops(int(pc.seq_lens[0]) - n_new, n_new, pc.q.shape[1], pc.head_dim)
        tf = fl / (float(np.mean(us)) * 1e-6) / 1e12
        result["prefill_hd256"] = {
            "workload": "head_dim-256 chunked prefill: 8,192 new on a 32,768-token fp8 "
                        "cache, 8/4 heads, causal, per-token-head scales",
            **stats(us), "flops": fl,
            "roofline": {"bound": "mfma", "achieved": round(tf, 1), "peak": FP8_PEAK_TFLOPS,
                         "unit": "TFLOP/s", "frac": round(tf / FP8_PEAK_TFLOPS, 4),
                         "kernel": "prefill_kernel"}}
        # the two-level ablation: the same launch with level 2 as an explicit float32
        # VALU flush per 64-key chunk instead of the MFMA's chained C operand
        us_v = timer.run(lambda i: kvq.prefill_attention(c, pq, pcu, pbt, psl, n_new, ones,
                                                         out=out, accumulation="valu_add"),
                         10, 3, warm_ms=200.0)
        tf_v = fl / (float(np.mean(us_v)) * 1e-6) / 1e12
        result["prefill_hd256_valu_add"] = {
            "workload": "the same prefill, level-2 accumulation as float32 VALU adds of a "
                        "zeroed accumulator per 64-key chunk (kvq_prefill_attention_accum)",
            **stats(us_v), "frac_fp8_peak": round(tf_v / FP8_PEAK_TFLOPS, 4),
            "time_vs_mfma_chain": round(float(np.mean(us_v)) / float(np.mean(us)), 3)}
        del c
        torch.cuda.empty_cache()
        mr = mfma_ceiling(torch, dev)
        if mr is not None:
            result["prefill_hd256"]["mfma_ceiling"] = {
                **mr, "prefill_frac_of_measured": round(tf / mr["TFLOP_s"], 4)}

    for leg, (Hq_, Hkv_, D_) in (("prefill_d128", (32, 8, 128)), ("prefill_d64", (64, 8, 64))):
        if leg not in legs:
            continue
        # Llama-3.1-8B- / gpt-oss-20b-shaped chunked prefill: 8,192 new queries on a
        # 32,768-token fp8 cache (per-token-head scales), causal
        pc = workloads.make_prefill_case(106, [32768], [8192], Hq_, Hkv_, D_,
                                         table="identity", name=leg)
        log(f"bench: {leg} workload generated")
        c = kvq.PagedCache(pc.num_pages, pc.num_kv_heads, pc.head_dim, "fp8", "per_token_head")
        for t0 in range(0, len(pc.k), 16384):
            sl_ = slice(t0, t0 + 16384)
            kvq.cache_write(c, to_dev(pc.k[sl_]), to_dev(pc.v[sl_]),
                            torch.from_numpy(pc.slots[sl_].astype(np.int64)).to(dev))
        pq, pcu = to_dev(pc.q), torch.from_numpy(pc.cu_q_lens).to(dev)
        pbt, psl = torch.from_numpy(pc.block_table).to(dev), torch.from_numpy(pc.seq_lens).to(dev)
        n_new = int(pc.cu_q_lens[1])
        out = torch.empty(pc.q.shape, dtype=torch.bfloat16, device=dev)
        us = timer.run(lambda i: kvq.prefill_attention(c, pq, pcu, pbt, psl, n_new, ones,
                                                       out=out), 10, 3, warm_ms=200.0)
        fl = prefill_flops(int(pc.seq_lens[0]) - n_new, n_new, Hq_, D_)
        tf = fl / (float(np.mean(us)) * 1e-6) / 1e12
        result[leg] = {
            "workload": f"head_dim-{D_} chunked prefill: 8,192 new on a 32,768-token fp8 "
                        f"cache, {Hq_}/{Hkv_} heads, causal, per-token-head scales",
            **stats(us), "flops": fl,
            "roofline": {"bound": "mfma", "achieved": round(tf, 1), "peak": FP8_PEAK_TFLOPS,
                         "unit": "TFLOP/s", "frac": round(tf / FP8_PEAK_TFLOPS, 4),
                         "kernel": "prefill_kernel"}}
        del c, pc
        torch.cuda.empty_cache()

    if "prefill_bf16_window" in legs:
        # gpt-oss-20b-shaped sliding-window layer prefill over its bf16 cache: 8,192 new
        # queries on a 32,768-token context, 64/8 heads, D 64, window 128, causal
        pc = workloads.make_prefill_case(107, [32768], [8192], 64, 8, 64, table="identity",
                                         window=128, name="bf16 window prefill")
        c = kvq.PagedCache(pc.num_pages, 8, 64, "bf16", "per_tensor")
        for t0 in range(0, len(pc.k), 16384):
            sl_ = slice(t0, t0 + 16384)
            kvq.cache_write(c, to_dev(pc.k[sl_]), to_dev(pc.v[sl_]),
                            torch.from_numpy(pc.slots[sl_].astype(np.int64)).to(dev))
        pq, pcu = to_dev(pc.q), torch.from_numpy(pc.cu_q_lens).to(dev)
        pbt, psl = torch.from_numpy(pc.block_table).to(dev), torch.from_numpy(pc.seq_lens).to(dev)
        out = torch.empty(pc.q.shape, dtype=torch.bfloat16, device=dev)
        us = timer.run(lambda i: kvq.prefill_attention(c, pq, pcu, pbt, psl, 8192, ones,
                                                       window=128, out=out), 10, 3, warm_ms=200.0)
        fl = 4.0 * 64 * 64 * 8192 * 128      # every query sees 128 keys
        tf = fl / (float(np.mean(us)) * 1e-6) / 1e12
        result["prefill_bf16_window"] = {
            "workload": "gpt-oss-20b-shaped window-128 layer prefill over its bf16 cache: "
                        "8,192 new on 32,768 ctx, 64/8 heads, D 64",
            **stats(us), "flops": fl,
            "roofline": {"bound": "mfma", "achieved": round(tf, 1), "peak": BF16_PEAK_TFLOPS,
                         "unit": "TFLOP/s", "frac": round(tf / BF16_PEAK_TFLOPS, 4),
                         "kernel": "prefill_bf16_kernel"}}
        del c, pc
        torch.cuda.empty_cache()

    if "per_kv_head" in legs:
        # the Llama-shaped decode step with per-KV-head scale arrays instead of
        # per-token-head scales (the same inputs; 8 random head scales per pool)
        case2 = workloads.llama8b_decode()
        last2 = case2.last_token_rows()
        hist2 = np.setdiff1d(np.arange(len(case2.k)), last2)
        hk = (0.004 * 2.0 ** np.random.default_rng(5).uniform(0, 5, 8)).astype(np.float32)
        hv = (0.004 * 2.0 ** np.random.default_rng(6).uniform(0, 5, 8)).astype(np.float32)
        cs = [kvq.PagedCache(case2.num_pages, 8, 128, "fp8", "per_kv_head",
                             k_head_scales=hk, v_head_scales=hv) for _ in range(args.rotate)]
        for i in range(0, len(hist2), 16384):
            sel = hist2[i:i + 16384]
            kk, vv = to_dev(case2.k[sel]), to_dev(case2.v[sel])
            ss = torch.from_numpy(case2.slots[sel].astype(np.int64)).to(dev)
            for c in cs:
                kvq.cache_write(c, kk, vv, ss)
        q2, kn2, vn2 = to_dev(case2.q), to_dev(case2.k[last2]), to_dev(case2.v[last2])
        bt2, sl2 = (torch.from_numpy(case2.block_table).to(dev),
                    torch.from_numpy(case2.seq_lens).to(dev))
        L2 = int(case2.seq_lens[0])
        ws2 = kvq.decode_workspace(cs[0], 8, 32, L2, 0, 0, dev)
        out2 = torch.empty((8, 32, 128), dtype=torch.bfloat16, device=dev)

        def pstep(i):
            kvq.decode_step(cs[i % len(cs)], q2, kn2, vn2, bt2, sl2, L2, ones, out=out2,
                            workspace=ws2)
        for i in range(args.warmup):
            pstep(i)
        torch.cuda.synchronize()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record()
        for i in range(args.steps):
            pstep(i)
        e1.record()
        torch.cuda.synchronize()
        us2 = e0.elapsed_time(e1) * 1e3 / args.steps
        nb2 = decode_bytes(8, L2, 8, 32, 128, 1, 0) + write_bytes(8, 8, 128, 1, 0)
        result["per_kv_head_decode_step"] = {
            "workload": "Llama-shaped decode step (8 x 20,000, 32/8 heads, D 128) with "
                        "per-KV-head scale arrays",
            "us_per_step": round(us2, 2), "bytes": nb2,
            "GB_s": round(nb2 / (us2 * 1e-6) / 1e9, 1),
            "frac_hbm": round(nb2 / (us2 * 1e-6) / 1e9 / HBM_PEAK_GBS, 4)}
        del cs
        torch.cuda.empty_cache()

    if "paged_logits" in legs:
        # sparse-attention indexer scores: 32 requests x 20,000 cached tokens, one query
        # row each, 4 query heads on one key head, D 128, fp8 per-token-head cache (the
        # indexer shape of the pages' test, at a serving batch and context)
        B3, L3 = 32, 20000
        lc = workloads.make_logits_case(109, [L3] * B3, [1] * B3, 4, 1, 128, table="perm",
                                        name="paged logits")
        # at least 8 copies (8 x 84.5 MB): with 4, the three others plus the output
        # (~264 MB) are about what the 256 MB last-level cache holds, and a launch
        # measured ~3% fast
        cs = [kvq.PagedCache(lc.num_pages, 1, 128, "fp8", "per_token_head")
              for _ in range(max(8, args.rotate))]
        for i in range(0, len(lc.k), 65536):
            sl_ = slice(i, i + 65536)
            kk, vv = to_dev(lc.k[sl_]), to_dev(lc.v[sl_])
            ss = torch.from_numpy(lc.slots[sl_].astype(np.int64)).to(dev)
            for c in cs:
                kvq.cache_write(c, kk, vv, ss)
        lq = to_dev(lc.q)
        lcu, lrl = torch.from_numpy(lc.cu_rows).to(dev), torch.from_numpy(lc.row_lens).to(dev)
        lbt, lsl = (torch.from_numpy(lc.block_table).to(dev),
                    torch.from_numpy(lc.seq_lens).to(dev))
        lout = torch.empty((B3, 4, L3), dtype=torch.float32, device=dev)

        def lstep(i):
            kvq.paged_logits(cs[i % len(cs)], lq, lcu, lrl, lbt, lsl, L3, ones, out=lout)
        for i in range(args.warmup):
            lstep(i)
        torch.cuda.synchronize()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record()
        for i in range(args.steps):
            lstep(i)
        e1.record()
        torch.cuda.synchronize()
        us3 = e0.elapsed_time(e1) * 1e3 / args.steps
        # K codes and per-token scales read, float32 logits written (query and block
        # table are < 0.3%)
        nb3 = B3 * L3 * 128 + B3 * L3 * 4 + B3 * 4 * L3 * 4
        result["paged_logits"] = {
            "workload": "indexer logits: 32 requests x 20,000 cached tokens, 1 query row "
                        "each, 4 query heads / 1 key head, D 128, fp8 per-token-head; "
                        "float32 [32][4][20,000] out",
            "us_per_launch": round(us3, 2), "bytes": nb3,
            "GB_s": round(nb3 / (us3 * 1e-6) / 1e9, 1),
            "frac_hbm": round(nb3 / (us3 * 1e-6) / 1e9 / HBM_PEAK_GBS, 4),
            "timing": "HIP events around a burst of back-to-back launches over rotating "
                      "cache copies"}
        del cs, lout
        torch.cuda.empty_cache()
        # prefill-time selection: one request of 8,192 new rows (causal: row i sees i + 1
        # keys) over its 8,192 keys, same heads and cache; 1 GB of float32 scores, so
        # bound by HBM writes -- set beside a plain 1 GB fill on the same output
        R4 = L4 = 8192
        pc = workloads.make_logits_case(113, [L4], [R4], 4, 1, 128, table="perm",
                                        name="paged logits rows")
        c4 = kvq.PagedCache(pc.num_pages, 1, 128, "fp8", "per_token_head")
        kvq.cache_write(c4, to_dev(pc.k), to_dev(pc.v),
                        torch.from_numpy(pc.slots.astype(np.int64)).to(dev))
        pq = to_dev(pc.q)
        pcu, prl = torch.from_numpy(pc.cu_rows).to(dev), torch.from_numpy(pc.row_lens).to(dev)
        pbt, psl = (torch.from_numpy(pc.block_table).to(dev),
                    torch.from_numpy(pc.seq_lens).to(dev))
        pout = torch.empty((R4, 4, L4), dtype=torch.float32, device=dev)

        def timed(fn, n, warm):
            for _ in range(warm):
                fn()
            torch.cuda.synchronize()
            t0 = torch.cuda.Event(enable_timing=True)
            t1 = torch.cuda.Event(enable_timing=True)
            t0.record()
            for _ in range(n):
                fn()
            t1.record()
            torch.cuda.synchronize()
            return t0.elapsed_time(t1) * 1e3 / n
        n4 = max(5, min(args.steps, 40))
        # 100 launches (~25 ms) of warmup: over the first few tens of milliseconds of such
        # a write-heavy load the launch time climbs from ~225 to ~275 us and settles near
        # 215 us (the clock adjusting); the figure is the settled one
        us4 = timed(lambda: kvq.paged_logits(c4, pq, pcu, prl, pbt, psl, L4, ones, out=pout),
                    n4, 100)
        usf = timed(lambda: pout.fill_(0.0), n4, 3)
        nb4 = R4 * 4 * L4 * 4 + L4 * 132
        result["paged_logits"]["prefill_rows"] = {
            "workload": "1 request x 8,192 query rows (causal) x 8,192 cached tokens, 4 "
                        "query heads / 1 key head, D 128, fp8 per-token-head; float32 "
                        "[8,192][4][8,192] out",
            "us_per_launch": round(us4, 2), "bytes": nb4,
            "GB_s": round(nb4 / (us4 * 1e-6) / 1e9, 1),
            "frac_hbm": round(nb4 / (us4 * 1e-6) / 1e9 / HBM_PEAK_GBS, 4),
            "fill_1GB_GB_s": round(R4 * 4 * L4 * 4 / (usf * 1e-6) / 1e9, 1),
            "frac_of_fill": round(usf / us4, 4)}
        del c4, pout
        torch.cuda.empty_cache()

    if "prefill_split" in legs:
        # short query chunks on a long context (keys split over workgroups, then merged):
        # one sequence of 131,072 cached tokens, Llama-shaped heads (32/8, D 128),
        # fp8 per-token-head; 16 and 256 new tokens, split and unsplit
        Ls = 131072
        npg = Ls // 16
        gen = torch.Generator(device=dev)
        gen.manual_seed(41)
        bts = torch.randperm(npg, device=dev, generator=gen).to(torch.int32).reshape(1, -1)
        cs_ = kvq.PagedCache(npg, 8, 128, "fp8", "per_token_head")
        pos = torch.arange(Ls, device=dev)
        sl_all = bts[0][pos // 16].to(torch.int64) * 16 + pos % 16
        for i in range(0, Ls, 65536):
            kk = torch.randn(65536, 8, 128, device=dev, generator=gen).to(torch.bfloat16)
            vv = torch.randn(65536, 8, 128, device=dev, generator=gen).to(torch.bfloat16)
            kvq.cache_write(cs_, kk, vv, sl_all[i:i + 65536])
        sls = torch.full((1,), Ls, device=dev, dtype=torch.int32)
        res_s = {"workload": "1 sequence, 131,072 cached tokens (the new ones last), 32/8 "
                             "heads, D 128, fp8 per-token-head, causal; keys split over "
                             "workgroups and merged (kvq_prefill_attention_ws) against "
                             "the unsplit kernel",
                 "timing": "HIP events over back-to-back launches after 3 untimed"}
        for n_new in (16, 256):
            qs = torch.randn(n_new, 32, 128, device=dev, generator=gen).to(torch.bfloat16)
            cus = torch.tensor([0, n_new], device=dev, dtype=torch.int32)
            outs_ = torch.empty_like(qs)
            row = {}
            for split in (True, False):
                def f():
                    kvq.prefill_attention(cs_, qs, cus, bts, sls, n_new, ones, out=outs_,
                                          split=split)
                for _ in range(3):
                    f()
                torch.cuda.synchronize()
                t0 = torch.cuda.Event(enable_timing=True)
                t1 = torch.cuda.Event(enable_timing=True)
                nrep = max(5, min(args.steps, 30))
                t0.record()
                for _ in range(nrep):
                    f()
                t1.record()
                torch.cuda.synchronize()
                row["us_split" if split else "us_unsplit"] = round(
                    t0.elapsed_time(t1) * 1e3 / nrep, 1)
            row["speedup"] = round(row["us_unsplit"] / row["us_split"], 2)
            res_s[f"new_{n_new}"] = row
        result["prefill_split"] = res_s
        del cs_
        torch.cuda.empty_cache()

    if "cache_write" in legs:
        # the quantising cache write in its bulk form: the Llama-shaped layer's whole
        # cache (160,000 tokens x 8 KV heads, D 128, per-token-head scales) and the
        # head_dim-256 prefill chunk's 8,192 new tokens (4 KV heads, per-token-head)
        cw = {}
        # (the third: the same fill with every 16-token block starting two tokens into a
        # page, as when a chunk begins mid-page)
        for name, (T, Hkv_, D_, shift) in (("llama8b_fill", (160000, 8, 128, 0)),
                                            ("hd256_new_tokens", (8192, 4, 256, 0)),
                                            ("llama8b_fill_mid_page", (160000, 8, 128, 2))):
            P_ = (T + shift + 15) // 16
            c = kvq.PagedCache(P_, Hkv_, D_, "fp8", "per_token_head")
            kk = dev_normal((T, Hkv_, D_), 1.0, 7000 + D_)
            vv = dev_normal((T, Hkv_, D_), 1.0, 7100 + D_)
            sl_ = torch.arange(shift, shift + T, dtype=torch.int64, device=dev)
            us = timer.run(lambda i: kvq.cache_write(c, kk, vv, sl_), 20, 3, warm_ms=100.0)
            nb = write_bytes(T, Hkv_, D_, 1, 8) + T * 8   # + the slot mapping
            cw[name] = {"tokens": T, "kv_heads": Hkv_, "head_dim": D_, "slot_shift": shift,
                        **stats(us),
                        "bytes": nb, "GB_s": round(nb / (float(np.mean(us)) * 1e-6) / 1e9, 1),
                        "frac_hbm": round(nb / (float(np.mean(us)) * 1e-6) / 1e9 / HBM_PEAK_GBS, 4)}
            del c, kk, vv
            torch.cuda.empty_cache()
        result["cache_write"] = {
            "workload": "quantising cache write, per-token-head scales, slots in page order "
                        "(bulk fill); bytes = bf16 K/V read + e4m3 codes and scales written "
                        "+ slot mapping", **cw}

    if "itl" in legs:
        log("bench: inter-token-latency sweep")
        result["itl_sweep"] = itl_sweep(list(ITL_CONTEXTS))

    if args.copy_calib:
        src = torch.empty(COPY_BYTES, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        result["copy_calib_bytes"] = COPY_BYTES

    if args.cpu_seqs > 0 and "decode" in legs:
        log("bench: timing the CPU oracle sample")
        result["cpu_baseline"] = cpu_baseline(workloads.llama8b_decode(),
                                              min(args.cpu_seqs, 8), args.cpu_reps)
    elif "decode" in legs:
        result["cpu_baseline"] = None
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
