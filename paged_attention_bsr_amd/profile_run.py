"""rocprofv3 runs of bench.py and their summaries (the files under profiles/).

    python -m paged_attention_bsr_amd.profile_run WORKLOAD [WORKLOAD ...] \
        [--out DIR] [--counters] [--steps K]

For each workload (a bench.py --workload name) this runs, from the
repository root, each as a child process under its own time limit:

  1. bench.py itself (its JSON line: value, roofline, HIP-event times);
  2. rocprofv3 --kernel-trace --stats over the same bench.py command
     (per-kernel launch durations);
  3. with --counters: three rocprofv3 --pmc passes of SQ counters (MFMA busy
     cycles, VALU / MFMA / LDS instructions, LDS bank conflicts, issue and
     wait cycles, GRBM_GUI_ACTIVE) and one pass each of FETCH_SIZE and
     WRITE_SIZE, the latter two with bench.py's --calibration-copy: a plain
     256 MiB device copy whose counter readings give the factor from the
     counters' units to bytes.

It then writes DIR/<kernel>_<workload>.md (the commands, the kernel
statistics, the bench line, the counters and derived rates) and merges
the HBM traffic per launch into DIR/traffic.json, keyed by workload with
the hash of the kernel's sources (bench.py reports it only while the
sources are unchanged).  The Python process running this never touches
the GPU itself.
"""
from __future__ import annotations

import argparse
import csv
import glob
import json
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

# counter passes that fit the per-block limits of one rocprofv3 --pmc run (<= 8 SQ, 2 GRBM)
SQ_PASSES = [
    "SQ_WAVES SQ_BUSY_CYCLES SQ_VALU_MFMA_BUSY_CYCLES SQ_INSTS_VALU SQ_INSTS_MFMA SQ_INSTS_LDS "
    "SQ_LDS_BANK_CONFLICT GRBM_GUI_ACTIVE",
    "SQ_WAIT_INST_LDS SQ_ACTIVE_INST_LDS SQ_ACTIVE_INST_VALU SQ_ACTIVE_INST_ANY SQ_WAIT_ANY SQ_WAVE_CYCLES "
    "SQ_VALU_MFMA_COEXEC_CYCLES SQ_INSTS_SALU",
    "SQ_INSTS_VALU_MFMA_MOPS_BF16 SQ_INSTS_VALU_MFMA_MOPS_F16 SQ_LDS_ADDR_CONFLICT SQ_LDS_UNALIGNED_STALL "
    "SQ_INSTS_LDS_LOAD_BANDWIDTH SQ_INSTS_LDS_STORE_BANDWIDTH SQ_INST_LEVEL_LDS SQ_BUSY_CU_CYCLES",
]
CALIB_MIB = 256
COPY_KERNEL = "__amd_rocclr_copyBuffer"
NUM_XCD, NUM_CU, SIMD_PER_CU = 8, 256, 4


def say(msg: str) -> None:
    print(msg, flush=True)


def run(cmd: list, limit: int, log_path: str, kill_first: bool = False) -> str:
    """Run cmd under `timeout` (SIGKILL straight away for counter passes), stdout
    returned, stderr to log_path; raises on a non-zero status."""
    lim = ["timeout", "-s", "KILL", str(limit)] if kill_first else ["timeout", "-k", "10", str(limit)]
    say("[profile] " + " ".join(cmd))
    log_path = os.path.join(ROOT, log_path)
    with open(log_path, "w") as err:
        proc = subprocess.run(lim + cmd, cwd=ROOT, stdout=subprocess.PIPE, stderr=err, text=True)
    if proc.returncode != 0:
        tail = open(log_path).read()[-2000:]
        raise RuntimeError(f"status {proc.returncode}: {' '.join(cmd)}\n{tail}")
    return proc.stdout


def bench_cmd(workload: str, steps: int, warmup: int, extra=()) -> list:
    return ["python3", "bench.py", "--workload", workload, "--steps", str(steps), "--warmup", str(warmup), *extra]


def last_json(text: str) -> dict:
    for line in reversed(text.strip().splitlines()):
        line = line.strip()
        if line.startswith("{"):
            return json.loads(line)
    raise RuntimeError("bench.py printed no JSON line")


def kernel_stats(d: str) -> list:
    paths = glob.glob(os.path.join(ROOT, d, "**", "*kernel_stats.csv"), recursive=True)
    if not paths:
        raise RuntimeError(f"no kernel statistics under {d}")
    return list(csv.DictReader(open(paths[0])))


def counters(d: str) -> dict:
    """{kernel name: {counter: mean per dispatch, '_dur_ns': mean dispatch duration}}."""
    paths = glob.glob(os.path.join(ROOT, d, "**", "*counter_collection.csv"), recursive=True)
    if not paths:
        raise RuntimeError(f"no counter collection under {d}")
    per: dict = {}
    seen = set()
    for r in csv.DictReader(open(paths[0])):
        k = r["Kernel_Name"]
        e = per.setdefault(k, {"_n": {}, "_dur": []})
        c = r["Counter_Name"]
        e.setdefault(c, 0.0)
        e[c] += float(r["Counter_Value"])
        e["_n"][c] = e["_n"].get(c, 0) + 1
        if (r["Dispatch_Id"], k) not in seen:
            seen.add((r["Dispatch_Id"], k))
            e["_dur"].append(int(r["End_Timestamp"]) - int(r["Start_Timestamp"]))
    out = {}
    for k, e in per.items():
        n, dur = e.pop("_n"), e.pop("_dur")
        out[k] = {c: v / n[c] for c, v in e.items()}
        out[k]["_dur_ns"] = sum(dur) / max(len(dur), 1)
    return out


def last_dispatch(d: str, kernel: str, counter: str) -> float:
    """The counter's value on the last dispatch of ``kernel`` in the run (the calibration
    copy comes after the timed loop; earlier copies of the same blit kernel move the inputs)."""
    paths = glob.glob(os.path.join(ROOT, d, "**", "*counter_collection.csv"), recursive=True)
    best, val = -1, None
    for r in csv.DictReader(open(paths[0])):
        if kernel in r["Kernel_Name"] and r["Counter_Name"] == counter and int(r["Dispatch_Id"]) > best:
            best, val = int(r["Dispatch_Id"]), float(r["Counter_Value"])
    if val is None:
        raise RuntimeError(f"no {kernel} dispatch with {counter} under {d}")
    return val


def pick(per: dict, kernel: str) -> dict:
    hits = [v for k, v in per.items() if kernel in k]
    if not hits:
        raise RuntimeError(f"{kernel} not found among {list(per)}")
    return hits[0]


def commands(workload: str, out: str, steps: int, with_counters: bool) -> list:
    """(kind, output dir or None, command) of every run, in order."""
    runs = [("bench", None, bench_cmd(workload, steps, 5))]
    d = os.path.join(out, f"trace_{workload}")
    runs.append(("trace", d, ["rocprofv3", "--kernel-trace", "--stats", "--output-format", "csv", "-d", d, "-o",
                              "run", "--", *bench_cmd(workload, steps, 5, ["--cpu-budget", "0"])]))
    if with_counters:
        short = ["--warm-s", "0", "--cpu-budget", "0"]
        for i, p in enumerate(SQ_PASSES):
            d = os.path.join(out, f"pmc_{workload}_sq{i + 1}")
            runs.append(("sq", d, ["rocprofv3", "--pmc", *p.split(), "--output-format", "csv", "-d", d, "-o", "run",
                                   "--", *bench_cmd(workload, 5, 2, short)]))
        for ctr in ("FETCH_SIZE", "WRITE_SIZE"):
            d = os.path.join(out, f"pmc_{workload}_{ctr}")
            runs.append((ctr, d, ["rocprofv3", "--pmc", ctr, "--output-format", "csv", "-d", d, "-o", "run", "--",
                                  *bench_cmd(workload, 5, 2, short + ["--calibration-copy", str(CALIB_MIB)])]))
    return runs


def profile(workload: str, out: str, steps: int, with_counters: bool, execute: bool = True) -> None:
    """Run the passes (unless ``execute`` is False: then summarise what an earlier
    run left in ``out``) and write the summary and traffic entry."""
    from bench import kernel_source_hash  # the hash bench.py checks the traffic entries against

    os.makedirs(os.path.join(ROOT, out), exist_ok=True)
    runs = commands(workload, out, steps, with_counters)
    bench_json = os.path.join(ROOT, out, f"bench_{workload}.json")
    line = stats = None
    sq, tr = {}, {}
    for kind, d, c in runs:
        if kind == "bench":
            if execute:
                line = last_json(run(c, 600, os.path.join(out, f"bench_{workload}.err")))
                json.dump(line, open(bench_json, "w"))
            line = json.load(open(bench_json))
            kernel = line["roofline"]["kernel"]
            say(f"[profile] {workload}: {line['value']:.1f} {line['unit']}, {kernel} "
                f"frac {line['roofline']['frac']:.3f}")
            continue
        if execute:
            run(c, 600 if kind == "trace" else 150, d + ".err", kill_first=kind != "trace")
        if kind == "trace":
            stats = kernel_stats(d)
        elif kind == "sq":
            sq.update(pick(counters(d), kernel))
        else:
            per = counters(d)
            copy_kib = last_dispatch(d, COPY_KERNEL, kind)
            tr[kind] = (pick(per, kernel)[kind], (CALIB_MIB << 10) / copy_kib, copy_kib)
        say(f"[profile] {workload}: {kind} pass done")
    traffic = None
    if tr:
        fetch_b = tr["FETCH_SIZE"][0] * tr["FETCH_SIZE"][1] * 1024
        write_b = tr["WRITE_SIZE"][0] * tr["WRITE_SIZE"][1] * 1024
        traffic = {"kernel": kernel, "kernel_source_hash": kernel_source_hash(kernel),
                   "fetch_kib_counted": tr["FETCH_SIZE"][0], "write_kib_counted": tr["WRITE_SIZE"][0],
                   "fetch_scale": tr["FETCH_SIZE"][1], "write_scale": tr["WRITE_SIZE"][1],
                   "copy_fetch_kib": tr["FETCH_SIZE"][2], "copy_write_kib": tr["WRITE_SIZE"][2],
                   "hbm_bytes_per_launch": fetch_b + write_b}
        tpath = os.path.join(ROOT, out, "traffic.json")
        data = json.load(open(tpath)) if os.path.exists(tpath) else {}
        data[workload] = traffic
        json.dump(data, open(tpath, "w"), indent=1, sort_keys=True)
    write_summary(workload, out, kernel, line, stats, sq, traffic, [" ".join(c) for _, _, c in runs])


def write_summary(workload, out, kernel, line, stats, sq, traffic, cmds) -> None:
    roof = line["roofline"]
    L = [f"# {kernel} on {workload}", "",
         f"Workload: {json.dumps(line['config'])}", "",
         "Made by `python -m paged_attention_bsr_amd.profile_run " + workload +
         (" --counters" if sq else "") + "`, which runs, from the repository root on one MI355X:", "", "```",
         *cmds, "```", "", "## rocprofv3 kernel statistics (--kernel-trace --stats)", "",
         "| kernel | calls | avg us | min us | max us | total % |", "|---|---|---|---|---|---|"]
    trace_avg = None
    for r in stats:
        name = r["Name"].replace("void ", "").replace("bsa::(anonymous namespace)::", "").replace("(bsa::AttnArgs)", "")
        L.append(f"| {name[:90]} | {r['Calls']} | {float(r['AverageNs']) / 1e3:.2f} | {float(r['MinNs']) / 1e3:.2f} | "
                 f"{float(r['MaxNs']) / 1e3:.2f} | {float(r['Percentage']):.1f} |")
        if kernel in r["Name"] and trace_avg is None:
            trace_avg = float(r["AverageNs"]) / 1e3
    L += ["", "## bench.py (HIP events on the launch stream, same command without the profiler)", "",
          f"- value: {line['value']:.1f} {line['unit']} (ms/step {line['ms_per_step']:.4f})",
          f"- roofline: bound {roof['bound']}, achieved {roof['achieved']:.1f} of {roof['peak']:.1f} {roof['unit']}, "
          f"frac {roof['frac']:.3f} ({roof.get('timing', '')})"]
    if "attention_ms_median" in roof:
        L.append(f"- attention kernel alone, median per step: {roof['attention_ms_median'] * 1e3:.2f} us; "
                 f"frac {roof.get('frac_attention_only', float('nan')):.3f}")
    if trace_avg is not None:
        per_launch = roof.get("alg_flops_per_launch") if roof["unit"] == "TFLOP/s" else roof.get("alg_bytes_per_launch")
        scale = 1e12 if roof["unit"] == "TFLOP/s" else 1e9
        if per_launch:
            ach = per_launch / (trace_avg * 1e-6) / scale
            L.append(f"- by the kernel-trace average ({trace_avg:.2f} us): {ach:.1f} {roof['unit']}, "
                     f"frac {ach / roof['peak']:.3f}")
    if line.get("cpu_baseline"):
        L.append(f"- cpu_baseline: {json.dumps(line['cpu_baseline'])}")
    if sq:
        dur = sq["_dur_ns"]
        cyc = sq.get("GRBM_GUI_ACTIVE", 0.0) / NUM_XCD
        L += ["", "## SQ counters of the kernel (rocprofv3 --pmc, mean per dispatch)", "",
              "| counter | value |", "|---|---|"]
        L += [f"| {k} | {v:.6g} |" for k, v in sorted(sq.items()) if not k.startswith("_")]
        L += ["", "Derived (GRBM_GUI_ACTIVE is summed over the 8 XCDs, so cycles = GRBM_GUI_ACTIVE / 8):", ""]
        if cyc > 0:
            L.append(f"- clock over the dispatch: {cyc / dur:.3f} GHz ({cyc:.0f} cycles in {dur / 1e3:.1f} us)")
            if "SQ_VALU_MFMA_BUSY_CYCLES" in sq:
                L.append(f"- MFMA busy: SQ_VALU_MFMA_BUSY_CYCLES / (cycles x 256 CUs x 4 SIMDs) = "
                         f"{sq['SQ_VALU_MFMA_BUSY_CYCLES'] / (cyc * NUM_CU * SIMD_PER_CU):.3f}")
            if "SQ_LDS_BANK_CONFLICT" in sq:
                L.append(f"- LDS bank-conflict cycles per CU cycle: "
                         f"{sq['SQ_LDS_BANK_CONFLICT'] / (cyc * NUM_CU):.4f}")
        if sq.get("SQ_WAVES"):
            w = sq["SQ_WAVES"]
            for c in ("SQ_INSTS_VALU", "SQ_INSTS_MFMA", "SQ_INSTS_LDS", "SQ_INSTS_SALU"):
                if c in sq:
                    L.append(f"- {c} per wave: {sq[c] / w:.1f}")
        if sq.get("SQ_ACTIVE_INST_VALU") and "SQ_VALU_MFMA_COEXEC_CYCLES" in sq:
            L.append(f"- VALU issue cycles overlapping MFMA: SQ_VALU_MFMA_COEXEC_CYCLES / SQ_ACTIVE_INST_VALU = "
                     f"{sq['SQ_VALU_MFMA_COEXEC_CYCLES'] / sq['SQ_ACTIVE_INST_VALU']:.3f}")
        if sq.get("SQ_WAVE_CYCLES") and "SQ_WAIT_INST_LDS" in sq:
            L.append(f"- share of wave cycles waiting on LDS instructions: "
                     f"{sq['SQ_WAIT_INST_LDS'] / sq['SQ_WAVE_CYCLES']:.3f}")
    if traffic:
        alg = roof.get("alg_bytes_per_launch", 0)
        L += ["", "## HBM traffic of the kernel (rocprofv3 --pmc, one pass per counter)", "",
              f"- FETCH_SIZE: {traffic['fetch_kib_counted']:.0f} KiB counted per dispatch; "
              f"WRITE_SIZE: {traffic['write_kib_counted']:.0f} KiB",
              f"- calibration: a {CALIB_MIB} MiB device copy ({COPY_KERNEL}, the run's last dispatch of it) reads "
              f"{traffic['copy_fetch_kib']:.0f} KiB on FETCH_SIZE and writes {traffic['copy_write_kib']:.0f} KiB "
              f"on WRITE_SIZE, so the counts are scaled by {traffic['fetch_scale']:.3f} and {traffic['write_scale']:.3f}",
              (f"- HBM bytes per launch: {traffic['hbm_bytes_per_launch'] / 1e6:.1f} MB; algorithmic bytes "
               f"{alg / 1e6:.1f} MB (ratio {traffic['hbm_bytes_per_launch'] / alg if alg else float('nan'):.3f})"
               if roof["bound"] == "hbm" else
               f"- HBM bytes per launch: {traffic['hbm_bytes_per_launch'] / 1e6:.1f} MB (the roofline of this "
               f"kernel is in flops; its byte count, K and V once per query row and kv head, is not a floor for "
               f"a tiled kernel)"),
              f"- kernel source hash: {traffic['kernel_source_hash']}"]
    path = os.path.join(ROOT, out, f"{kernel}_{workload}.md")
    with open(path, "w") as f:
        f.write("\n".join(L) + "\n")
    say(f"[profile] wrote {path}")


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("workloads", nargs="+")
    ap.add_argument("--out", default=os.path.join("gpurun_out", "prof"))
    ap.add_argument("--counters", action="store_true")
    ap.add_argument("--steps", type=int, default=150)
    ap.add_argument("--summarize-only", action="store_true",
                    help="write the summaries from what an earlier run left in --out (no GPU work)")
    args = ap.parse_args()
    out = os.path.relpath(args.out, ROOT) if os.path.isabs(args.out) else args.out  # children run in ROOT
    for wl in args.workloads:
        profile(wl, out, args.steps, args.counters, execute=not args.summarize_only)
    return 0


if __name__ == "__main__":
    sys.exit(main())
