"""Build libbsa.so in-tree with hipcc for gfx950.

    python -m paged_attention_bsr_amd.build          # build both libraries (always recompiles)

Host-only sources (the planner) are compiled with the host compiler, HIP
sources with hipcc for --offload-arch=gfx950, then linked into
paged_attention_bsr_amd/libbsa.so.  Packed-FP32 VALU instructions are
disabled for all device code (-packed-fp32-ops).

The same sources built with -DBSA_TRACE give libbsa_trace.so, whose
kernels also write per-tile trace records (bsa_trace_records); only tests
load it.
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
TRACE_LIB = os.path.join(PKG, "libbsa_trace.so")
BUILD_DIR = os.path.join(ROOT, "_build")

ARCH = os.environ.get("BSA_OFFLOAD_ARCH", "gfx950")
HIPCC = os.environ.get("HIPCC", shutil.which("hipcc") or "/opt/rocm/bin/hipcc")

COMMON = ["-O3", "-fPIC", "-std=c++17", "-I", INCLUDE, "-I", CSRC, "-Wall", "-Wno-unused-function"]
HIP_FLAGS = [f"--offload-arch={ARCH}", "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
             "-ffp-contract=fast", "-munsafe-fp-atomics"]
# Extra -D definitions for tuning builds (e.g. "-DBSA_DECODE_NW=2"); empty for the product build.
EXTRA = os.environ.get("BSA_EXTRA_CFLAGS", "").split()

HIP_SOURCES = ["attn_tile.hip", "attn_decode.hip", "attn_mla.hip", "merge.hip", "rope_quant.hip", "indexer.hip",
               "api.cpp"]
HOST_SOURCES = ["planner.cpp", "abi_host.cpp"]


def _run(cmd):
    proc = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    out = "\n".join(l for l in proc.stdout.splitlines()
                    if "packed-fp32-ops" not in l and "unused during compilation" not in l)
    if proc.returncode != 0:
        raise RuntimeError(f"command failed ({proc.returncode}): {' '.join(cmd)}\n{out}")
    return out


def _variant_jobs(build_dir: str, defs: list) -> list:
    jobs = []
    for src in HIP_SOURCES:
        obj = os.path.join(build_dir, src + ".o")
        lang = ["-x", "hip"] if src.endswith(".cpp") else []
        jobs.append([HIPCC, *COMMON, *HIP_FLAGS, *EXTRA, *defs, *lang, "-c", os.path.join(CSRC, src), "-o", obj])
    for src in HOST_SOURCES:
        obj = os.path.join(build_dir, src + ".o")
        jobs.append(["g++", *COMMON, *EXTRA, *defs, "-c", os.path.join(CSRC, src), "-o", obj])
    return jobs


def build(verbose: bool = False, trace: bool = True) -> str:
    """Compile every source and link libbsa.so (and, with ``trace``, libbsa_trace.so);
    returns the product library's path."""
    variants = [(LIB, BUILD_DIR, [])]
    if trace:
        variants.append((TRACE_LIB, os.path.join(BUILD_DIR, "trace"), ["-DBSA_TRACE"]))
    jobs = []
    for _, bdir, defs in variants:
        os.makedirs(bdir, exist_ok=True)
        jobs.append(_variant_jobs(bdir, defs))
    with ThreadPoolExecutor(max_workers=8) as ex:
        outs = list(ex.map(_run, [j for vj in jobs for j in vj]))
    if verbose:
        for o in outs:
            if o.strip():
                print(o)
    for (lib_path, _, _), vj in zip(variants, jobs):
        objs = [j[-1] for j in vj]
        tmp = lib_path + ".tmp"
        _run([HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs])
        os.replace(tmp, lib_path)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv, trace="--no-trace" not in sys.argv))
