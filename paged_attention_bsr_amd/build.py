"""Build libbsa.so in-tree with hipcc for gfx950.

    python -m paged_attention_bsr_amd.build          # build (always recompiles)

Host-only sources (the planner) are compiled with the host compiler, HIP
sources with hipcc for --offload-arch=gfx950, then linked into
paged_attention_bsr_amd/libbsa.so.  Packed-FP32 VALU instructions are
disabled for all device code (-packed-fp32-ops).
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libbsa.so")
BUILD_DIR = os.path.join(ROOT, "_build")

ARCH = os.environ.get("BSA_OFFLOAD_ARCH", "gfx950")
HIPCC = os.environ.get("HIPCC", shutil.which("hipcc") or "/opt/rocm/bin/hipcc")

COMMON = ["-O3", "-fPIC", "-std=c++17", "-I", INCLUDE, "-I", CSRC, "-Wall", "-Wno-unused-function"]
HIP_FLAGS = [f"--offload-arch={ARCH}", "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
             "-ffp-contract=fast", "-munsafe-fp-atomics"]
# Extra -D definitions for tuning builds (e.g. "-DBSA_DECODE_NW=2"); empty for the product build.
EXTRA = os.environ.get("BSA_EXTRA_CFLAGS", "").split()

HIP_SOURCES = ["attn_tile.hip", "attn_decode.hip", "attn_mla.hip", "merge.hip", "rope_quant.hip", "api.cpp"]
HOST_SOURCES = ["planner.cpp"]


def _run(cmd):
    proc = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    out = "\n".join(l for l in proc.stdout.splitlines()
                    if "packed-fp32-ops" not in l and "unused during compilation" not in l)
    if proc.returncode != 0:
        raise RuntimeError(f"command failed ({proc.returncode}): {' '.join(cmd)}\n{out}")
    return out


def build(verbose: bool = False) -> str:
    """Compile every source and link libbsa.so; returns the library path."""
    os.makedirs(BUILD_DIR, exist_ok=True)
    jobs = []
    for src in HIP_SOURCES:
        obj = os.path.join(BUILD_DIR, src + ".o")
        lang = ["-x", "hip"] if src.endswith(".cpp") else []
        jobs.append([HIPCC, *COMMON, *HIP_FLAGS, *EXTRA, *lang, "-c", os.path.join(CSRC, src), "-o", obj])
    for src in HOST_SOURCES:
        obj = os.path.join(BUILD_DIR, src + ".o")
        jobs.append(["g++", *COMMON, *EXTRA, "-c", os.path.join(CSRC, src), "-o", obj])
    with ThreadPoolExecutor(max_workers=min(8, len(jobs))) as ex:
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
    print(build(verbose="-v" in sys.argv))
