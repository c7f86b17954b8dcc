#!/usr/bin/env python3
"""Benchmark of BSR block-sparse attention on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload all|NAME]

A step is one run of the planned attention (attention kernel, plus the LSE
merge kernel when the plan splits rows) over one batch of synthetic inputs
already resident in HBM.  Planning (host) and the one-time table upload are
done before the timed region and reported separately (plan_ms).

By default the five configurations of the headline metric run one after the
other (worked example, paged decode, block-sparse prefill, windowed prefill,
sparse MLA); ONE JSON line is printed, whose headline is the paged-decode
figure and whose ``configs`` array holds one entry per configuration.  For
the decode workloads the metric is KV GB/s (algorithmic bytes: K and V of
every unmasked key once per kv head, plus q, o, lse and the index
structure); for the block-sparse prefill workloads it is TFLOP/s
(algorithmic flops: 4 * head_dim * qo heads * unmasked query-key pairs).
``roofline`` divides the algorithmic work by the median GPU time of a step
(attention + merge kernels, HIP events on the launch stream) over the timed
steps; ``cpu_baseline`` times the CPU oracle on a bounded sample of the same
workload on this host's cores.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
METRIC = "KV GB/s (decode) & TFLOP/s (sparse prefill), % of MI355X HBM/MFMA peak"
HBM_PEAK_GBS = 8000.0
MFMA_PEAK_TFLOPS = {"f16": 2516.6, "bf16": 2516.6}
DECODE = {"paged_decode", "sparse_mla", "worked_example", "paged_decode_fp8"}
# sources of each attention kernel (the traffic counters are valid while these are unchanged)
KERNEL_SOURCES = {
    "attn_tile_kernel": ["attn_tile.hip", "device_common.h", "kernels.h"],
    "attn_decode_kernel": ["attn_decode.hip", "device_common.h", "kernels.h"],
    "attn_mla_kernel": ["attn_mla.hip", "device_common.h", "kernels.h"],
    "rope_quant_kernel": ["rope_quant.hip", "rope_quant.h", "device_common.h"],
    "indexer_scores_kernel": ["indexer.hip", "indexer.h", "device_common.h"],
}


def log(msg: str) -> None:
    print(msg, file=sys.stderr, flush=True)


def kernel_source_hash(kernel: str) -> str:
    h = hashlib.sha256()
    for f in KERNEL_SOURCES[kernel]:
        with open(os.path.join(ROOT, "paged_attention_bsr_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def head_structures(w):
    """The (indptr, indices) rows of each structure head: one shared BSR, or one per kv
    head for a per-head block mask (``w.meta["block_mask"]``)."""
    import numpy as np
    bm = w.meta.get("block_mask")
    if bm is None:
        return [(w.indptr, w.indices)]
    out = []
    for h in range(bm.shape[0]):
        rows = [np.nonzero(bm[h, I])[0] for I in range(bm.shape[1])]
        out.append((np.cumsum([0] + [len(r) for r in rows]), np.concatenate(rows).astype(np.int32)))
    return out


def unmasked_pairs(w, rows=None, indptr=None, indices=None):
    """Unmasked (query row, key) pairs of one structure (the shared BSR unless given),
    counted block by block."""
    import numpy as np
    indptr = w.indptr if indptr is None else indptr
    indices = w.indices if indices is None else indices
    lens = w.kv_block_lens
    off = w.N - w.M
    row_set = None if rows is None else np.asarray(sorted(rows))
    total = 0
    for I in range(len(indptr) - 1):
        r0, r1 = I * w.R, min(w.M, (I + 1) * w.R)
        rr = np.arange(r0, r1)
        if row_set is not None:
            rr = rr[np.isin(rr, row_set)]
            if rr.size == 0:
                continue
        for J in indices[indptr[I]:indptr[I + 1]]:
            n = w.C if lens is None else int(lens[J])
            if not w.causal:
                total += n * rr.size
            else:
                allowed = np.clip(rr + off - int(J) * w.C + 1, 0, n)
                total += int(allowed.sum())
    return total


def masked_kv_pairs(w, rows=None):
    """Visible (query row, key) pairs summed over kv heads for element masks
    (``w.meta["mask"]``, shared by every kv head) or variable blocks
    (``w.meta["variable"]``, one map per kv head); None for other workloads."""
    import numpy as np
    row_list = np.arange(w.M) if rows is None else np.asarray(sorted(rows))
    if "mask" in w.meta:
        mask = w.meta["mask"]
        total = 0
        for I in range(len(w.indptr) - 1):
            sel = row_list[(row_list >= I * w.R) & (row_list < (I + 1) * w.R)] - I * w.R
            if sel.size:
                total += int(mask[w.indptr[I]:w.indptr[I + 1]][:, sel, :].sum())
        return total * w.num_kv_heads
    if "variable" in w.meta:
        bm, rs, cs = w.meta["variable"]
        total = 0
        for h in range(bm.shape[0]):
            row_block = np.repeat(np.arange(bm.shape[1]), rs[h])
            c_end = np.cumsum(cs[h])
            c_start = c_end - cs[h]
            if not w.causal:
                keys = (bm[h] * cs[h][None, :]).sum(axis=1)
                total += int(keys[row_block[row_list]].sum())
            else:
                for i in row_list:
                    lim = i + w.N - w.M + 1
                    vis = np.clip(np.minimum(c_end, lim) - c_start, 0, None)
                    total += int((bm[h, row_block[i]] * vis).sum())
        return total
    return None


def algorithmic_work(w, rows=None):
    """(bytes, flops) the method itself must move / compute for one run (or for `rows` only).

    bytes: K and V of every unmasked key once per (query row, kv head) -- for
    the decode shapes (R = 1) that is each selected cache row once -- (for
    the latent MLA cache one 576-value row per key, V being its prefix),
    plus q, o, lse and the int32 index structure.
    flops: 2 * (head_dim + head_dim_vo) per unmasked pair and qo head
    (QK^T and PV).
    """
    structs = head_structures(w)
    # pairs summed over kv heads (a shared structure counts once per kv head)
    masked = masked_kv_pairs(w, rows)
    if masked is not None:
        kv_pairs = masked
    elif len(structs) == 1:
        kv_pairs = unmasked_pairs(w, rows) * w.num_kv_heads
    else:
        kv_pairs = sum(unmasked_pairs(w, rows, ip, ix) for ip, ix in structs)
    g = w.num_qo_heads // w.num_kv_heads
    m = w.M if rows is None else len(rows)
    e_kv = w.kv_dtype.itemsize
    if w.v_aliases_k:
        kv_bytes = kv_pairs * w.head_dim * e_kv
    else:
        kv_bytes = kv_pairs * (w.head_dim + w.head_dim_vo) * e_kv
    qo = m * w.num_qo_heads * (w.head_dim * w.q_dtype.itemsize + w.head_dim_vo * w.o_dtype.itemsize + 4)
    idx = 0
    for ip, ix in structs:
        nnz_rows = len(ix) if rows is None else sum(int(ip[r // w.R + 1] - ip[r // w.R]) for r in rows)
        idx += 4 * (m + 1 + nnz_rows)
        if w.kv_block_lens is not None:
            idx += 4 * nnz_rows
    flops = 2 * kv_pairs * g * (w.head_dim + w.head_dim_vo)
    scale_bytes = sum(4 * len(w.meta[f"scale_{n}"]) for n in ("q", "k", "v") if f"scale_{n}" in w.meta)
    if "mask" in w.meta:   # the element masks, one bit each, for the rows taken
        idx += w.meta["mask"].size // 8 * m // w.M
    if "variable" in w.meta:   # the block map (one bit per block) and the int32 sizes
        bm, rs, cs = w.meta["variable"]
        idx += bm.size // 8 + 4 * (rs.size + cs.size)
    return kv_bytes + qo + idx + scale_bytes, flops


def cpu_baseline(w, budget_s: float):
    """Time the CPU oracle, as it stands, on a bounded sample of query rows of the same workload."""
    import numpy as np
    import oracle
    import torch
    try:
        from threadpoolctl import threadpool_info
        threads = max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        threads = os.cpu_count() or 1
    if w.kv_dtype == torch.float8_e4m3fn and not w.v_aliases_k:
        k = oracle.fp8_dequant(w.k.view(torch.uint8).numpy(), w.meta.get("scale_k"), w.k_descale)
        v = oracle.fp8_dequant(w.v.view(torch.uint8).numpy(), w.meta.get("scale_v"), w.v_descale)
    elif w.kv_dtype == torch.float8_e4m3fn:
        kf = oracle.e4m3fn_decode(w.k.view(torch.uint8).numpy())
        k = (kf * w.k_descale)[:, None, :]
        v = (kf[:, :w.head_dim_vo] * w.v_descale)[:, None, :]
    else:
        k, v = w.k.double().numpy(), w.v.double().numpy()
    q = w.q.double().numpy()
    if "scale_q" in w.meta:
        q = q * w.meta["scale_q"].astype(np.float64)[None, :, None]
    order = np.random.default_rng(0).permutation(w.M)
    done, t_used, batch = 0, 0.0, 1
    while done < w.M and t_used < budget_s:
        rows = order[done:done + batch].tolist()
        t0 = time.perf_counter()
        if "variable" in w.meta:
            bm, rs, cs = w.meta["variable"]
            oracle.variable_block_attention(bm, rs, cs, q, k, v, sm_scale=w.sm_scale, causal=w.causal, rows=rows)
        elif "mask" in w.meta:
            oracle.element_mask_attention(w.indptr, w.indices, w.M, w.N, w.R, w.C, w.meta["mask"], q, k, v,
                                          sm_scale=w.sm_scale, rows=rows)
        elif "block_mask" in w.meta:
            oracle.block_mask_attention(w.meta["block_mask"], w.M, w.N, w.R, w.C, q, k, v,
                                        sm_scale=w.sm_scale, causal=w.causal,
                                        kv_block_lens=w.kv_block_lens, rows=rows)
        else:
            oracle.bsr_attention(w.indptr, w.indices, w.M, w.N, w.R, w.C, q, k, v, sm_scale=w.sm_scale,
                                 causal=w.causal, kv_block_lens=w.kv_block_lens, rows=rows)
        t_used += time.perf_counter() - t0
        done += len(rows)
        batch = min(batch * 2, 64)
    b, f = algorithmic_work(w, order[:done].tolist())
    return {"seconds": t_used, "rows": done, "bytes": b, "flops": f, "cores": threads}


# The five configurations of the headline metric, in order; the JSON line's
# headline is the paged-decode one (the metric's decode figure), and every
# one of them gets an entry in its "configs" array.
CONFIGS = ["worked_example", "paged_decode", "bsr_prefill", "window_prefill", "sparse_mla"]
HEADLINE = "paged_decode"


def host_cores():
    """(os.cpu_count(), CPUs this process may run on, BLAS threads in use)."""
    try:
        affinity = len(os.sched_getaffinity(0))
    except (AttributeError, OSError):  # pragma: no cover
        affinity = os.cpu_count() or 1
    try:
        from threadpoolctl import threadpool_info
        blas = max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        blas = affinity
    return os.cpu_count() or 1, affinity, blas


# Steps per pair of timing events: a HIP event pair costs a few microseconds of GPU
# time on this part (outside the pair's own window, so the wall clock of the timed
# region carries it), so each pair brackets CHUNK consecutive steps and the step's
# GPU time is the pair's elapsed time / CHUNK (one sample per chunk).
CHUNK = 25
# Default seconds of warm-up work (at least --warmup steps) before a workload's timed region.
WARM_S = 0.25


def timed_chunks(fn, steps: int):
    """Run fn() ceil(steps / CHUNK) * CHUNK times, bracketing every CHUNK calls with HIP events
    on torch's current stream (the stream the library launches on).  Returns the wall
    time of the whole region and the GPU milliseconds per call of every chunk."""
    import torch
    n = max(1, -(-steps // CHUNK))
    events = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(n)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for e0, e1 in events:
        e0.record()
        for _ in range(CHUNK):
            fn()
        e1.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    return wall, [e0.elapsed_time(e1) / CHUNK for e0, e1 in events]


def measure(name: str, args, dev):
    """Plan, upload, warm up and time one workload; returns (its entry of the JSON line, the workload).

    A step is bsa_run (attention kernel, then the merge kernel when rows are split).
    Its GPU time comes from HIP events around chunks of CHUNK steps; the roofline
    fraction uses the median over the chunks.  The attention kernel alone is timed
    the same way in a second loop (bsa_run_phase)."""
    import numpy as np
    import torch
    from paged_attention_bsr_amd import Plan
    from paged_attention_bsr_amd import _lib as L
    from paged_attention_bsr_amd import workloads as W

    t0 = time.perf_counter()
    w = W.by_name(name)
    gen_s = time.perf_counter() - t0
    kv_splits = W.BENCH_KV_SPLITS[name] if args.kv_splits is None else args.kv_splits
    t0 = time.perf_counter()
    if "variable" in w.meta:
        bm, rs, cs = w.meta["variable"]
        plan = Plan.variable(bm, rs, cs, w.num_qo_heads, w.num_kv_heads, w.head_dim, causal=w.causal,
                             sm_scale=w.sm_scale, kv_splits=kv_splits, q_dtype=w.q_dtype,
                             R=args.var_grid[0], C=args.var_grid[1])
    else:
        plan = Plan(w.indptr, w.indices, w.M, w.N, w.R, w.C, w.num_qo_heads, w.num_kv_heads, w.head_dim,
                    head_dim_vo=w.head_dim_vo, causal=w.causal, sm_scale=w.sm_scale, kv_splits=kv_splits,
                    kv_block_lens=w.kv_block_lens, q_dtype=w.q_dtype, kv_dtype=w.kv_dtype, o_dtype=w.o_dtype,
                    k_descale=w.k_descale, v_descale=w.v_descale, k_token_stride=w.k_token_stride,
                    v_token_stride=w.v_token_stride, block_mask=w.meta.get("block_mask"),
                    packed_mask=w.meta.get("packed_mask"))
    plan_ms = (time.perf_counter() - t0) * 1e3
    info = plan.info()
    q = w.q.to(dev)
    k = w.k.to(dev)
    v = None if w.v_aliases_k else w.v.to(dev)
    out = torch.empty((w.M, w.num_qo_heads, w.head_dim_vo), dtype=w.o_dtype, device=dev)
    lse = torch.empty((w.M, w.num_qo_heads), dtype=torch.float32, device=dev)
    ws = plan.workspace(dev)
    plan.upload(ws)
    torch.cuda.synchronize()
    log(f"[bench] {name}: inputs {gen_s:.1f} s, plan {plan_ms:.1f} ms: {info}")

    # per-head run() scales (fp8 KV workloads), device float32
    scales = {f"scale_{n}": torch.from_numpy(w.meta[f"scale_{n}"]).to(dev)
              for n in ("q", "k", "v") if f"scale_{n}" in w.meta}

    # the arguments are validated once (Plan.bind): a step is then only the bsa_run_ex call,
    # so host overhead does not leave the GPU idle between launches
    step, _, _ = plan.bind(q, k, v, out=out, lse=lse, workspace=ws, **scales)
    attention_only, _, _ = plan.bind(q, k, v, out=out, lse=lse, workspace=ws, phase=L.BSA_PHASE_ATTENTION,
                                     **scales)

    # W warm-up steps, continued until the GPU has been busy for WARM_S (its clocks come up
    # from idle, e.g. after the previous workload's host work)
    def warm_up(fn, min_calls):
        calls, t_w = 0, time.perf_counter()
        while calls < min_calls or time.perf_counter() - t_w < args.warm_s:
            fn()
            calls += 1
            if calls % 8 == 0:
                torch.cuda.synchronize()
        torch.cuda.synchronize()
        return calls

    warm_steps = warm_up(step, args.warmup)
    wall, step_ms = timed_chunks(step, args.steps)
    ms_per_step = wall * 1e3 / len(step_ms) / CHUNK
    gpu_ms = float(np.median(step_ms))
    # the attention-only loop gets a warm-up of its own: after the synchronisation that
    # ends the timed steps the clocks may have dropped again
    warm_up(attention_only, args.warmup)
    _, attn_ms = timed_chunks(attention_only, args.steps)
    attn_med = float(np.median(attn_ms))
    step()   # leave a complete result behind
    torch.cuda.synchronize()
    log(f"[bench] {name}: {len(step_ms) * CHUNK} steps: {ms_per_step:.4f} ms/step wall; GPU step (attention + "
        f"merge) median {gpu_ms:.4f} ms, mean {float(np.mean(step_ms)):.4f}; attention kernel median {attn_med:.4f} ms")
    del q, k, v, out, lse, ws, scales
    torch.cuda.empty_cache()

    if args.calibration_copy > 0:
        n = args.calibration_copy << 20
        src = torch.ones(n, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        log(f"[bench] calibration copy: {n} bytes read, {n} bytes written")
        del src, dst

    alg_bytes, alg_flops = algorithmic_work(w)
    decode = name in DECODE
    kernel = {L.BSA_KERNEL_MLA: "attn_mla_kernel", L.BSA_KERNEL_DECODE: "attn_decode_kernel"}.get(
        info["kernel"], "attn_tile_kernel")
    if decode:
        value = alg_bytes / (ms_per_step * 1e-3) / 1e9
        unit = "GB/s"
        achieved = alg_bytes / (gpu_ms * 1e-3) / 1e9
        roof = {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": achieved / HBM_PEAK_GBS}
    else:
        value = alg_flops / (ms_per_step * 1e-3) / 1e12
        unit = "TFLOP/s"
        achieved = alg_flops / (gpu_ms * 1e-3) / 1e12
        peak = MFMA_PEAK_TFLOPS["f16" if w.q_dtype == torch.float16 else "bf16"]
        roof = {"bound": "mfma", "achieved": achieved, "peak": peak, "unit": "TFLOP/s", "frac": achieved / peak}
    if name == "worked_example":
        roof["bound_note"] = "launch latency: 5 key blocks, 81,920 flop; a parity configuration"
    if name == "sparse_mla":
        # exact bf16 MFMA arithmetic bounds this shape too; report its MFMA fraction beside HBM
        roof["mfma_frac_bf16"] = alg_flops / (gpu_ms * 1e-3) / 1e12 / MFMA_PEAK_TFLOPS["bf16"]
    roof["traffic"] = measured_traffic(name, kernel_source_hash(kernel))
    roof["kernel"] = kernel
    roof["timing"] = (f"median over {len(step_ms)} chunks of {CHUNK} steps of the HIP-event GPU time per step "
                      "(attention + merge kernels)")
    roof["step_gpu_ms_median"] = gpu_ms
    roof["attention_ms_median"] = attn_med
    roof["alg_bytes_per_launch"] = alg_bytes
    roof["alg_flops_per_launch"] = alg_flops
    roof["frac_attention_only"] = roof["frac"] * gpu_ms / attn_med if attn_med > 0 else None

    dtype = {torch.float16: "f16", torch.bfloat16: "bf16"}[w.q_dtype]
    if w.kv_dtype == torch.float8_e4m3fn:
        dtype = f"{dtype} (fp8 e4m3 KV storage)"
    cfg = {"workload": name, "M": w.M, "N": w.N, "R": info["R"], "C": info["C"],
           "num_qo_heads": w.num_qo_heads, "num_kv_heads": w.num_kv_heads, "head_dim": w.head_dim,
           "head_dim_vo": w.head_dim_vo, "causal": w.causal,
           "nnz_blocks": sum(len(ix) for _, ix in head_structures(w)),
           "per_head_structure": "block_mask" in w.meta or "variable" in w.meta,
           "element_masks": "mask" in w.meta or "variable" in w.meta, "kv_splits": kv_splits,
           "tiles": info["num_tiles"], "merges": info["num_merges"], "plan_ms": plan_ms,
           "alg_bytes": alg_bytes, "alg_flops": alg_flops}
    cfg["warmup_steps_run"] = warm_steps
    return {"workload": name, "metric": METRIC, "value": value, "unit": unit, "ms_per_step": ms_per_step,
            "dtype": dtype, "config": cfg, "roofline": roof, "cpu_baseline": None}, w


def cpu_entry(w, unit: str, budget_s: float) -> dict:
    """The CPU oracle, as it stands, timed on a bounded sample of the workload, in the metric's unit."""
    log(f"[bench] {w.name}: CPU oracle baseline (~{budget_s:.0f} s budget)")
    cb = cpu_baseline(w, budget_s)
    cval = (cb["bytes"] / 1e9 if unit == "GB/s" else cb["flops"] / 1e12) / cb["seconds"]
    n_cpu, n_aff, n_blas = host_cores()
    return {"value": cval, "unit": unit, "cores": n_blas, "os_cpu_count": n_cpu, "affinity_cores": n_aff,
            "blas_threads": n_blas, "kind": "oracle",
            "sample": f"{cb['rows']} of {w.M} query rows (all heads), float64 dense-mask oracle, "
                      f"{cb['seconds']:.1f} s"}


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=500, help="timed steps (rounded up to a multiple of 25)")
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="all",
                    choices=["all", "worked_example", "paged_decode", "bsr_prefill", "window_prefill", "sparse_mla",
                             "head_sparse_prefill", "paged_decode_fp8", "element_mask_prefill",
                             "variable_block_prefill", "bsr_prefill_fp8", "rope_quantize", "indexer"],
                    help="all = the five configurations (headline: paged_decode); otherwise one workload")
    ap.add_argument("--warm-s", type=float, default=WARM_S,
                    help="keep warming up (beyond --warmup steps) until the GPU has worked this many seconds")
    ap.add_argument("--kv-splits", type=int, default=None, help="override the workload's split-KV setting")
    ap.add_argument("--var-grid", type=int, nargs=2, default=(0, 0), metavar=("R", "C"),
                    help="variable-block workloads: the fixed grid the blocks are mapped onto (0 = library's choice)")
    ap.add_argument("--cpu-budget", type=float, default=8.0,
                    help="seconds of CPU oracle work per workload (0 = skip)")
    ap.add_argument("--calibration-copy", type=int, default=0, metavar="MIB",
                    help="after each timed region, copy MIB MiB device-to-device once (a known-size "
                         "reference for rocprofv3 FETCH_SIZE / WRITE_SIZE counters)")
    args = ap.parse_args()
    args.steps = max(CHUNK, -(-args.steps // CHUNK) * CHUNK)   # whole chunks of timed steps

    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (got --gpus {args.gpus}): the library has no multi-GPU path; "
              "the attention would shard by kv head or by request with no exchange between GPUs.", file=sys.stderr)
        return 2

    import torch
    sys.path.insert(0, ROOT)

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        return 1
    dev = torch.device("cuda", 0)
    torch.cuda.set_device(dev)
    props = torch.cuda.get_device_properties(dev)
    log(f"[bench] device {props.name} CUs={props.multi_processor_count} workload={args.workload}")

    if args.workload == "rope_quantize":
        return run_rope_quantize(args, dev)
    if args.workload == "indexer":
        return run_indexer(args, dev)

    names = CONFIGS if args.workload == "all" else [args.workload]
    # every GPU measurement first (back to back, the GPU kept busy), then the host baselines
    measured = [measure(n, args, dev) for n in names]
    entries = []
    for e, w in measured:
        if args.cpu_budget > 0:
            e["cpu_baseline"] = cpu_entry(w, e["unit"], args.cpu_budget)
        entries.append(e)
    del measured
    head = next(e for e in entries if e["workload"] == (HEADLINE if args.workload == "all" else args.workload))
    line = {"metric": METRIC, "value": head["value"], "unit": head["unit"], "n_gpus": 1, "steps": args.steps,
            "warmup": args.warmup, "ms_per_step": head["ms_per_step"], "higher_is_better": True,
            "scaling": "weak", "vs_baseline": None, "dtype": head["dtype"], "data": "synthetic",
            "config": head["config"], "roofline": head["roofline"], "cpu_baseline": head["cpu_baseline"],
            "configs": [{k: e[k] for k in ("workload", "value", "unit", "ms_per_step", "dtype", "roofline",
                                           "cpu_baseline", "config")} for e in entries]}
    print(json.dumps(line), flush=True)
    return 0


def rope_bytes(nnz: int, heads: int) -> int:
    """Algorithmic bytes of the RoPE + FP8 quantize producer for nnz tokens: the bf16 q
    (heads x 576) and k (576) rows read, their fp8 codes written, the int32 position and
    the token's 64-value fp32 cache row read."""
    return nnz * (heads * 576 * 3 + 576 * 3 + 4 + 256)


def run_rope_quantize(args, dev) -> int:
    """One step = one bsa_mla_rope_quantize_fp8 over the workload's token chunk."""
    import numpy as np
    import torch
    from paged_attention_bsr_amd import mla_rope_quantize_fp8
    from paged_attention_bsr_amd import workloads as W
    w = W.rope_quantize()
    nnz, H = w["nnz"], w["num_heads"]
    d = {k: w[k].to(dev) for k in ("q_rope", "k_rope", "q_nope", "k_nope", "cos_sin_cache", "pos_ids")}
    f8 = torch.float8_e4m3fn
    outs = {"q_rope_out": torch.empty(nnz, H, 64, dtype=f8, device=dev),
            "k_rope_out": torch.empty(nnz, 64, dtype=f8, device=dev),
            "q_nope_out": torch.empty(nnz, H, 512, dtype=f8, device=dev),
            "k_nope_out": torch.empty(nnz, 512, dtype=f8, device=dev)}

    def step():
        mla_rope_quantize_fp8(d["q_rope"], d["k_rope"], d["q_nope"], d["k_nope"], d["cos_sin_cache"], d["pos_ids"],
                              w["is_neox"], w["quant_scale_q"], w["quant_scale_kv"], **outs)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    events = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(args.steps)]
    t0 = time.perf_counter()
    for i in range(args.steps):
        events[i][0].record()
        step()
        events[i][1].record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_per_step = wall * 1e3 / args.steps
    k_ms = float(np.median([e[0].elapsed_time(e[1]) for e in events]))
    log(f"[bench] {args.steps} steps: {ms_per_step:.4f} ms/step; kernel median {k_ms:.4f} ms")
    if args.calibration_copy > 0:
        n = args.calibration_copy << 20
        src = torch.ones(n, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    alg = rope_bytes(nnz, H)
    achieved = alg / (k_ms * 1e-3) / 1e9
    roof = {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": achieved / HBM_PEAK_GBS,
            "kernel": "rope_quant_kernel", "traffic": measured_traffic("rope_quantize", kernel_source_hash("rope_quant_kernel")),
            "alg_bytes_per_launch": alg, "alg_flops_per_launch": 0, "step_gpu_ms_median": k_ms,
            "timing": "median of HIP-event kernel time over the timed steps"}
    cpu = None
    if args.cpu_budget > 0:
        import oracle
        log(f"[bench] CPU oracle baseline (~{args.cpu_budget:.0f} s budget)")
        n_cpu, n_aff, threads = host_cores()
        cache = w["cos_sin_cache"].float().numpy()
        done, used, batch = 0, 0.0, 8
        while done < nnz and used < args.cpu_budget:
            sl = slice(done, min(nnz, done + batch))
            f = lambda t: t[sl].float().numpy()
            t1 = time.perf_counter()
            oracle.mla_rope_quantize_fp8(f(w["q_rope"]), f(w["k_rope"]), f(w["q_nope"]), f(w["k_nope"]), cache,
                                         w["pos_ids"][sl].numpy(), w["is_neox"], w["quant_scale_q"],
                                         w["quant_scale_kv"])
            used += time.perf_counter() - t1
            done = sl.stop
            batch = min(batch * 2, 256)
        cpu = {"value": rope_bytes(done, H) / used / 1e9, "unit": "GB/s", "cores": threads, "os_cpu_count": n_cpu,
               "affinity_cores": n_aff, "blas_threads": threads, "kind": "oracle",
               "sample": f"{done} of {nnz} tokens (all heads), numpy float32 rotary + nearest-value fp8 encode, "
                         f"{used:.1f} s"}
    cfg = {"workload": "rope_quantize", "nnz": nnz, "num_heads": H, "q_row": "512 latent + 64 rope",
           "max_seq_len": w["max_seq_len"], "is_neox": w["is_neox"], "cache": "fp32",
           "quant_scale_q": w["quant_scale_q"], "quant_scale_kv": w["quant_scale_kv"], "alg_bytes": alg}
    line = {"metric": METRIC, "value": alg / (ms_per_step * 1e-3) / 1e9, "unit": "GB/s", "n_gpus": 1,
            "steps": args.steps, "warmup": args.warmup, "ms_per_step": ms_per_step, "higher_is_better": True,
            "scaling": "weak", "vs_baseline": None, "dtype": "bf16 in, fp8 e4m3 out (f32 arithmetic)",
            "data": "synthetic", "config": cfg, "roofline": roof, "cpu_baseline": cpu}
    print(json.dumps(line), flush=True)
    return 0


def indexer_bytes(w: dict) -> int:
    """Algorithmic bytes of one indexer step: each request's keys read once (up to its longest
    row's context), the query rows read and the int32 index lists written.  The float32 score
    rows are an intermediate of this implementation, not part of the floor."""
    rp, ctx, D = w["req_row_ptr"], w["ctx_len"], w["head_dim"]
    keys = sum(int(ctx[rp[r]:rp[r + 1]].max()) for r in range(w["num_reqs"]) if rp[r + 1] > rp[r])
    return keys * D * 2 + w["num_rows"] * D * 2 + w["num_rows"] * w["topk"] * 4


def indexer_scores_bytes(w: dict) -> int:
    """Algorithmic bytes of one launch of the scores kernel: each request's keys and the query
    rows read once, and the float32 score of every (row, position < n) written."""
    rp, ctx, D = w["req_row_ptr"], w["ctx_len"], w["head_dim"]
    keys = sum(int(ctx[rp[r]:rp[r + 1]].max()) for r in range(w["num_reqs"]) if rp[r + 1] > rp[r])
    n = sum(min(int(c), w["max_ctx"]) for c in ctx)
    return keys * D * 2 + w["num_rows"] * D * 2 + n * 4


def run_indexer(args, dev) -> int:
    """One step = one bsa_indexer_topk (scores kernel, then Top-K kernel) over the workload's
    query rows: the indexer upstream of the sparse-MLA configuration."""
    import numpy as np
    import torch
    from paged_attention_bsr_amd import indexer_topk
    from paged_attention_bsr_amd import workloads as W
    w = W.indexer()
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(dev)
    q, kc = w["q"].to(dev), w["key_cache"].to(dev)
    bt, rp, ctx, kv = t(w["block_table"]), t(w["req_row_ptr"]), t(w["ctx_len"]), t(w["req_kv_len"])
    rows, K = w["num_rows"], w["topk"]
    scores = torch.empty((rows, (w["max_ctx"] + 63) // 64 * 64), dtype=torch.float32, device=dev)
    out = torch.empty((rows, K), dtype=torch.int32, device=dev)

    def run(scores_only):
        return lambda: indexer_topk(q, kc, bt, rp, ctx, kv, K, w["page_size"], max_ctx=w["max_ctx"], scores=scores,
                                    out=out, scores_only=scores_only)

    step, scores_step = run(False), run(True)
    for fn in (step, scores_step):
        n, t_w = 0, time.perf_counter()
        while n < args.warmup or time.perf_counter() - t_w < args.warm_s:
            fn()
            n += 1
        torch.cuda.synchronize()
    wall, step_ms = timed_chunks(step, args.steps)
    ms_per_step = wall * 1e3 / len(step_ms) / CHUNK
    gpu_ms = float(np.median(step_ms))
    n, t_w = 0, time.perf_counter()
    while n < args.warmup or time.perf_counter() - t_w < args.warm_s:
        scores_step()
        n += 1
    torch.cuda.synchronize()
    _, sc_ms = timed_chunks(scores_step, args.steps)
    sc_med = float(np.median(sc_ms))
    step()
    torch.cuda.synchronize()
    log(f"[bench] indexer: {len(step_ms) * CHUNK} steps: {ms_per_step:.4f} ms/step wall; GPU step median "
        f"{gpu_ms:.4f} ms (scores kernel {sc_med:.4f} ms, the two Top-K kernels {gpu_ms - sc_med:.4f} ms)")
    if args.calibration_copy > 0:
        n = args.calibration_copy << 20
        src = torch.ones(n, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    alg = indexer_bytes(w)
    sc_alg = indexer_scores_bytes(w)
    flops = 2 * w["head_dim"] * int(np.asarray(w["ctx_len"], np.int64).sum())
    achieved = sc_alg / (sc_med * 1e-3) / 1e9
    step_ach = alg / (gpu_ms * 1e-3) / 1e9
    roof = {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": achieved / HBM_PEAK_GBS,
            "kernel": "indexer_scores_kernel",
            "traffic": measured_traffic("indexer", kernel_source_hash("indexer_scores_kernel")),
            "alg_bytes_per_launch": sc_alg, "alg_flops_per_launch": flops, "kernel_ms_median": sc_med,
            "step_gpu_ms_median": gpu_ms, "topk_kernels_ms": gpu_ms - sc_med, "step_alg_bytes": alg,
            "step_achieved": step_ach, "step_frac": step_ach / HBM_PEAK_GBS,
            "timing": f"scores kernel alone: median over {len(sc_ms)} chunks of {CHUNK} scores-only calls of the "
                      f"HIP-event GPU time per call; step: the same over {len(step_ms)} chunks of whole steps"}
    cpu = None
    if args.cpu_budget > 0:
        import oracle
        log(f"[bench] indexer: CPU oracle baseline (~{args.cpu_budget:.0f} s budget)")
        n_cpu, n_aff, threads = host_cores()
        qn, kn = w["q"].float().numpy(), w["key_cache"].float().numpy()
        done, used, done_bytes = 0, 0.0, 0
        while done < rows and used < args.cpu_budget:
            t1 = time.perf_counter()
            oracle.indexer_topk(qn[done:done + 1], kn, w["block_table"], w["page_size"], np.array([0, 1], np.int32),
                                w["ctx_len"][done:done + 1], K)
            used += time.perf_counter() - t1
            done_bytes += int(w["ctx_len"][done]) * w["head_dim"] * 2 + w["head_dim"] * 2 + K * 4
            done += 1
        cpu = {"value": done_bytes / used / 1e9, "unit": "GB/s", "cores": threads, "os_cpu_count": n_cpu,
               "affinity_cores": n_aff, "blas_threads": threads, "kind": "oracle",
               "sample": f"{done} of {rows} query rows, each reading its own keys, float64 scores + sort, "
                         f"{used:.1f} s"}
    cfg = {"workload": "indexer", "num_rows": rows, "num_reqs": w["num_reqs"], "head_dim": w["head_dim"],
           "topk": K, "page_size": w["page_size"], "num_slots": w["num_slots"], "max_ctx": w["max_ctx"],
           "alg_bytes": alg, "alg_flops": flops}
    line = {"metric": METRIC, "value": alg / (ms_per_step * 1e-3) / 1e9, "unit": "GB/s", "n_gpus": 1,
            "steps": args.steps, "warmup": args.warmup, "ms_per_step": ms_per_step, "higher_is_better": True,
            "scaling": "weak", "vs_baseline": None, "dtype": "bf16 in, f32 scores, int32 out",
            "data": "synthetic", "config": cfg, "roofline": roof, "cpu_baseline": cpu}
    print(json.dumps(line), flush=True)
    return 0


def measured_traffic(workload: str, src_hash: str):
    """HBM bytes per launch from the committed rocprofv3 counter summary, if it
    was taken on the current kernel sources; else None."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        data = json.load(f)
    ent = data.get(workload)
    if not ent or ent.get("kernel_source_hash") != src_hash:
        return None
    return ent.get("hbm_bytes_per_launch")


if __name__ == "__main__":
    sys.exit(main())
