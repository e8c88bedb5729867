"""Build libkvq.so (HIP for gfx950) in-tree: ``python -m fp8_quantized_paged_amd.build``.

Every source under csrc/ is compiled by hipcc for gfx950 only, with packed-fp32
instruction selection disabled, then linked into fp8_quantized_paged_amd/libkvq.so.
"""
from __future__ import annotations

import hashlib
import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
BUILD = os.path.join(HERE, "_build")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(HERE, "libkvq.so")
# measurement probe (bench.py only; not part of the library or its source hash)
PROBE_SRC = os.path.join(HERE, "probe", "mfma_rate.hip")
PROBE_LIB = os.path.join(HERE, "libkvq_probe.so")
ARCH = "gfx950"

SOURCES = ["host.cpp", "cache_write.hip", "decode.hip", "decode_noalloc.hip", "prefill.hip", "prefill_d64.hip",
           "prefill_d128.hip", "prefill_d256.hip", "prefill_bf16.hip", "logits.hip"]

COMMON_FLAGS = [
    "-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-unused-command-line-argument", "-Wno-inline-asm",
    # Keep the decode kernel's unrolled page ring: without this, SimplifyCFG sinks
    # the identical per-page code of the three buffers back into one block, which
    # removes the prefetch of the next pages.
    "-mllvm", "-simplifycfg-sink-common=false",
    f"-I{INCLUDE}", f"-I{CSRC}",
]


def source_hash() -> str:
    """SHA-256 (first 32 hex digits) of everything the library is built from: the
    sources, the public header and the compiler flags.  build() compiles it into the
    library (symbol kvq_build_source_hash); the binding refuses a library whose
    recorded hash differs from the tree's, i.e. a stale build."""
    h = hashlib.sha256()
    for name in sorted(os.listdir(CSRC)):
        if name.endswith((".hip", ".cpp", ".h")):
            h.update(name.encode() + b"\0")
            with open(os.path.join(CSRC, name), "rb") as f:
                h.update(f.read())
    with open(os.path.join(INCLUDE, "kvq.h"), "rb") as f:
        h.update(f.read())
    h.update(" ".join(COMMON_FLAGS[:-2]).encode())  # the -I paths depend on the checkout
    return h.hexdigest()[:32]


def hipcc() -> str:
    for cand in (shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found")


def build(verbose: bool = False, extra_flags=()) -> str:
    os.makedirs(BUILD, exist_ok=True)
    cc = hipcc()
    procs = []
    objs = []
    stamp = f'-DKVQ_SOURCE_HASH="{source_hash()}"'
    for src in SOURCES:
        path = os.path.join(CSRC, src)
        if not os.path.exists(path):
            continue
        obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
        objs.append(obj)
        cmd = [cc, "-c", path, "-o", obj, *COMMON_FLAGS, *extra_flags]
        if src == "host.cpp":
            cmd.append(stamp)
        if verbose:
            print(" ".join(cmd), flush=True)
        procs.append((src, subprocess.Popen(cmd, stdout=subprocess.PIPE,
                                            stderr=subprocess.STDOUT, text=True)))
    failed = []
    for src, p in procs:
        out, _ = p.communicate()
        out = "\n".join(line for line in out.splitlines()
                        if "packed-fp32-ops" not in line)
        if p.returncode != 0:
            failed.append((src, out))
        elif verbose and out.strip():
            print(out)
    if failed:
        msg = "\n\n".join(f"[{s}]\n{o}" for s, o in failed)
        raise RuntimeError(f"hipcc failed:\n{msg}")
    tmp = LIB + ".tmp"
    cmd = [cc, "-shared", "-fPIC", f"--offload-arch={ARCH}", *objs, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB)
    if os.path.exists(PROBE_SRC):
        cmd = [cc, "-shared", PROBE_SRC, "-o", PROBE_LIB + ".tmp", *COMMON_FLAGS, *extra_flags]
        if verbose:
            print(" ".join(cmd), flush=True)
        p = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
        if p.returncode != 0:
            raise RuntimeError(f"hipcc failed on the probe:\n{p.stdout}")
        os.replace(PROBE_LIB + ".tmp", PROBE_LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
