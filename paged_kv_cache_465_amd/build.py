"""Build libkvp.so (gfx950 kernels + host library) in-tree with hipcc.

    python -m paged_kv_cache_465_amd.build        # from the repository root

Objects go to _build/ at the repository root; the shared library lands next
to this file, where the Python binding loads it from.
"""
from __future__ import annotations

import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libkvp.so")
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")
HIPCC = os.path.join(ROCM, "bin", "hipcc")
ARCH = "gfx950"

# decode kernels: one translation unit per (KV format, plan), so they compile in parallel
DEVICE_SOURCES = [f"decode_{fmt}_{plan}.hip" for fmt in ("int4", "bf16", "fp8", "int8")
                  for plan in ("sched", "split")] + [f"prefill_{fmt}.hip" for fmt in ("int4", "bf16", "fp8", "int8")] \
    + ["prefill.hip", "decode.hip", "append.hip", "probe.hip"]
HOST_SOURCES = ["pool.cpp", "prefix_cache.cpp", "schedule.cpp"]

COMMON = ["-O3", "-std=c++17", "-fPIC", "-Wall", "-Wno-unused-result", f"-I{INCLUDE}", f"-I{CSRC}"]
# Device code: gfx950 only; packed-fp32 instructions off; IEEE-rounded fp32
# divide (the INT8 row contract depends on it); no fast-math anywhere.
DEVICE = [f"--offload-arch={ARCH}", "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
          "-fhip-fp32-correctly-rounded-divide-sqrt", "-ffp-contract=fast-honor-pragmas"]


def _run(cmd):
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    out = "\n".join(l for l in r.stdout.splitlines() if "unknown target feature" not in l
                    and "packed-fp32-ops" not in l)
    if r.returncode != 0:
        raise RuntimeError(f"command failed ({r.returncode}): {' '.join(cmd)}\n{out}")
    return out


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    jobs = []
    for src in DEVICE_SOURCES:
        obj = os.path.join(BUILD, src + ".o")
        jobs.append([HIPCC, *COMMON, *DEVICE, "-x", "hip", "-c", os.path.join(CSRC, src), "-o", obj])
    for src in HOST_SOURCES:
        obj = os.path.join(BUILD, src + ".o")
        # host-only C++ (no device code): compiled as plain C++
        jobs.append([HIPCC, *COMMON, "-x", "c++", "-c", os.path.join(CSRC, src), "-o", obj])
    with ThreadPoolExecutor(max_workers=min(8, os.cpu_count() or 4, len(jobs))) as ex:
        outs = list(ex.map(_run, jobs))
    if verbose:
        for o in outs:
            if o.strip():
                print(o)
    objs = [j[-1] for j in jobs]
    tmp = LIB + ".tmp"
    _run([HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs])
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    path = build(verbose="-v" in sys.argv)
    print(path)
