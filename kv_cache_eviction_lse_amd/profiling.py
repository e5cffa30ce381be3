"""Text summaries of rocprofv3 output for the eviction round (kernel statistics and the
scorer's HBM traffic), as kept under profiles/.

Kernel statistics (from `rocprofv3 --kernel-trace --stats --output-format csv`):

    python -m kv_cache_eviction_lse_amd.profiling stats --dir DIR --command "..." > summary.md

Socket power and graphics clock while a command runs (amd-smi samples):

    python -m kv_cache_eviction_lse_amd.profiling power --interval 0.5 -- python3 bench.py --hold 8

Matrix-core and vector-ALU activity of a kernel per launch, from one counter run
(SQ_VALU_MFMA_BUSY_CYCLES, SQ_INSTS_VALU_MFMA_MOPS_BF16, SQ_INSTS_MFMA, SQ_INSTS_VALU,
SQ_INSTS_VALU_TRANS_F32, SQ_ACTIVE_INST_VALU, SQ_VALU_MFMA_COEXEC_CYCLES,
SQ_BUSY_CU_CYCLES, GRBM_GUI_ACTIVE):

    python -m kv_cache_eviction_lse_amd.profiling compute --dir DIR --kernel score_mfma \
        --json out.json --command "..." > summary.md

HBM traffic of the scorer per launch, from two counter runs of bench.py with a plain
copy of known size (`--calibration-copy MiB`) in the same process: FETCH_SIZE and
WRITE_SIZE of each kernel are scaled by bytes / counter of the copy kernel.

    python -m kv_cache_eviction_lse_amd.profiling traffic --fetch DIR1 --write DIR2 \
        --copy-mib 2048 --json out.json --command "..." > summary.md
"""
from __future__ import annotations

import argparse
import csv
import glob
import hashlib
import json
import os
import re
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
SCORER = "score_mfma_kernel"


def _rows(directory: str, suffix: str) -> list[dict]:
    out = []
    for p in sorted(glob.glob(os.path.join(directory, "**", f"*{suffix}"), recursive=True)):
        with open(p, newline="") as f:
            out.extend(csv.DictReader(f))
    return out


def _short(name: str) -> str:
    name = re.sub(r"kvs::\(anonymous namespace\)::", "", name)
    name = name.replace("void ", "")
    return name.split("(")[0][:60]


def source_sha(name: str = "score.hip") -> str:
    p = os.path.join(HERE, "csrc", name)
    return hashlib.sha256(open(p, "rb").read()).hexdigest()[:16]


def score_source_sha() -> str:
    return source_sha("score.hip")


def stats(args) -> None:
    rows = _rows(args.dir, "kernel_stats.csv")
    if not rows:
        sys.exit(f"no kernel_stats.csv under {args.dir}")
    print("# Kernel time per launch (rocprofv3 kernel trace; kvs kernels only)\n")
    print(f"Command: `{args.command}`\n")
    print("| kernel | calls | average us | min us | max us | share of all GPU time |")
    print("|---|---|---|---|---|---|")
    for r in rows:
        nm = r["Name"]
        if "kvs::" not in nm and not args.all:
            continue
        print(f"| {_short(nm)} | {r['Calls']} | {float(r['AverageNs']) / 1e3:.1f} | "
              f"{float(r['MinNs']) / 1e3:.1f} | {float(r['MaxNs']) / 1e3:.1f} | {float(r['Percentage']):.1f} % |")


def _counter(directory: str, counter: str) -> dict[str, list[float]]:
    per = {}
    for r in _rows(directory, "counter_collection.csv"):
        if r.get("Counter_Name") != counter:
            continue
        per.setdefault(r["Kernel_Name"], []).append(float(r["Counter_Value"]))
    if not per:
        sys.exit(f"no {counter} rows under {directory}")
    return per


def _calibration_copies(directory: str, counter: str, n: int = 3) -> list[float]:
    """The counter values of the last n copy-kernel dispatches of the run: bench.py's
    --calibration-copy runs its copies after everything else."""
    rows = []
    for r in _rows(directory, "counter_collection.csv"):
        if r.get("Counter_Name") == counter and "copy" in r["Kernel_Name"].lower():
            rows.append((int(r.get("Dispatch_Id", 0) or 0), float(r["Counter_Value"])))
    rows.sort()
    return [v for _, v in rows[-n:]]


def traffic(args) -> None:
    kernel = args.kernel
    copy_bytes = args.copy_mib * 2**20
    out = {"kernel": kernel, "source_sha": source_sha(args.source), "source": args.source,
           "copy_bytes": copy_bytes}
    factors = {}
    for counter, d in (("FETCH_SIZE", args.fetch), ("WRITE_SIZE", args.write)):
        per = _counter(d, counter)
        # the calibration copy: the last copy dispatches of the run (other copies, such as
        # the per-step pool copies, come before it and have other sizes)
        copies = _calibration_copies(d, counter)
        if not copies:
            sys.exit(f"no copy kernel in the {counter} run")
        c_kib = max(copies)
        factor = copy_bytes / (c_kib * 1024.0)
        # every kernel whose name holds one of the '|'-separated substrings (template
        # names hold commas): the per-dispatch average of each, summed (one launch of
        # each per call)
        names = [k for k in per if any(x in k for x in kernel.split("|"))]
        if not names:
            sys.exit(f"no {kernel} dispatch in the {counter} run")
        s_kib = sum(sum(per[k]) / len(per[k]) for k in names)
        sc = [v for k in names for v in per[k]]
        key = counter.lower()
        out[f"{key}_kib_per_dispatch"] = s_kib
        out[f"copy_{key}_kib"] = c_kib
        out[f"{key}_factor"] = factor
        out[f"{key}_bytes_per_launch"] = s_kib * 1024.0 * factor
        out[f"{key}_dispatches"] = len(sc)
        factors[counter] = factor
    out["hbm_bytes_per_launch"] = out["fetch_size_bytes_per_launch"] + out["write_size_bytes_per_launch"]
    if args.algorithmic_bytes:
        out["algorithmic_bytes_per_launch"] = args.algorithmic_bytes
    out["commands"] = args.command
    with open(args.json, "w") as f:
        json.dump(out, f, indent=1)
    print(f"# {kernel}: HBM traffic per launch ({args.workload})\n")
    for c in args.command:
        print(f"Command: `{c}`\n")
    print("| counter | kernel KiB/dispatch | copy KiB ({} MiB copy) | bytes per counted byte | kernel bytes/launch |".format(args.copy_mib))
    print("|---|---|---|---|---|")
    for counter in ("FETCH_SIZE", "WRITE_SIZE"):
        k = counter.lower()
        print(f"| {counter} | {out[f'{k}_kib_per_dispatch']:.0f} | {out[f'copy_{k}_kib']:.0f} | "
              f"{out[f'{k}_factor']:.4f} | {out[f'{k}_bytes_per_launch']:.4e} |")
    print(f"\nHBM traffic per launch: {out['hbm_bytes_per_launch']:.4e} bytes", end="")
    if args.algorithmic_bytes:
        print(f" ({out['hbm_bytes_per_launch'] / args.algorithmic_bytes:.3f} x the algorithmic "
              f"{args.algorithmic_bytes:.4e})")
    else:
        print()
    print(f"\n{args.source} sha256[:16] = {out['source_sha']}")


COMPUTE_COUNTERS = ("SQ_VALU_MFMA_BUSY_CYCLES", "SQ_INSTS_VALU_MFMA_MOPS_BF16", "SQ_INSTS_MFMA", "SQ_INSTS_VALU",
                    "SQ_INSTS_VALU_TRANS_F32", "SQ_ACTIVE_INST_VALU", "SQ_VALU_MFMA_COEXEC_CYCLES",
                    "SQ_BUSY_CU_CYCLES", "GRBM_GUI_ACTIVE")
SIMDS, CUS, XCDS = 1024, 256, 8


def compute(args) -> None:
    """Per-launch averages of the compute counters of one kernel and the derived
    figures: MFMA busy = sum of per-SIMD MFMA busy cycles / (GPU active cycles x 1024
    SIMDs) (rocprofv3's MfmaUtil expression; GRBM_GUI_ACTIVE is summed over the 8 XCDs
    in the CSV, so it is divided by 8), bf16 MFMA flops = MOPS x 512."""
    avg = {}
    n = {}
    for c in COMPUTE_COUNTERS:
        per = _counter(args.dir, c)
        vals = [v for k, vs in per.items() if args.kernel in k for v in vs]
        if not vals:
            sys.exit(f"no {args.kernel} dispatch with {c}")
        avg[c] = sum(vals) / len(vals)
        n[c] = len(vals)
    gui = avg["GRBM_GUI_ACTIVE"] / XCDS
    out = {"kernel": args.kernel, "source": args.source, "source_sha": source_sha(args.source),
           "dispatches": min(n.values()), "counters_per_launch": avg,
           "gpu_active_cycles": gui,
           "mfma_busy_frac": avg["SQ_VALU_MFMA_BUSY_CYCLES"] / (gui * SIMDS),
           "mfma_bf16_flops": avg["SQ_INSTS_VALU_MFMA_MOPS_BF16"] * 512.0,
           "valu_per_mfma": avg["SQ_INSTS_VALU"] / max(avg["SQ_INSTS_MFMA"], 1.0),
           "trans_per_mfma": avg["SQ_INSTS_VALU_TRANS_F32"] / max(avg["SQ_INSTS_MFMA"], 1.0),
           "valu_busy_frac": avg["SQ_ACTIVE_INST_VALU"] / CUS / gui,
           "coexec_frac_of_mfma_busy": avg["SQ_VALU_MFMA_COEXEC_CYCLES"] / max(avg["SQ_VALU_MFMA_BUSY_CYCLES"], 1.0),
           "commands": args.command}
    if args.kernel_us:
        out["kernel_us"] = args.kernel_us
        out["clock_ghz_implied"] = gui / (args.kernel_us * 1e3)
        out["mfma_bf16_tflops"] = out["mfma_bf16_flops"] / (args.kernel_us * 1e-6) / 1e12
    with open(args.json, "w") as f:
        json.dump(out, f, indent=1)
    print(f"# {args.kernel}: matrix-core and vector-ALU counters per launch ({args.workload})\n")
    for c in args.command:
        print(f"Command: `{c}`\n")
    print(f"Dispatches averaged: {out['dispatches']}\n")
    print("| counter | per launch |")
    print("|---|---|")
    for c in COMPUTE_COUNTERS:
        print(f"| {c} | {avg[c]:.4e} |")
    print("\n| derived | value |")
    print("|---|---|")
    print(f"| GPU active cycles (GRBM_GUI_ACTIVE / 8 XCDs) | {gui:.4e} |")
    if args.kernel_us:
        print(f"| kernel time (trace) | {args.kernel_us:.1f} us |")
        print(f"| implied graphics clock | {out['clock_ghz_implied']:.2f} GHz |")
        print(f"| bf16 MFMA rate | {out['mfma_bf16_tflops']:.0f} TFLOP/s |")
    print(f"| MFMA busy (MFMA busy cycles / (active cycles x 1024 SIMDs)) | {out['mfma_busy_frac']:.3f} |")
    print(f"| bf16 MFMA flops (MOPS x 512) | {out['mfma_bf16_flops']:.4e} |")
    print(f"| VALU instructions per MFMA | {out['valu_per_mfma']:.2f} |")
    print(f"| fp32 transcendental instructions per MFMA | {out['trans_per_mfma']:.2f} |")
    print(f"| VALU busy (SQ_ACTIVE_INST_VALU / 256 CUs / active cycles) | {out['valu_busy_frac']:.3f} |")
    print(f"| co-issue cycles / MFMA busy cycles | {out['coexec_frac_of_mfma_busy']:.3f} |")
    print(f"\n{args.source} sha256[:16] = {out['source_sha']}")


def _smi_sample() -> tuple[float, float] | None:
    """(socket power W, first GFX clock MHz) from `amd-smi metric -p -c`, or None."""
    import subprocess
    try:
        txt = subprocess.run(["amd-smi", "metric", "-p", "-c"], capture_output=True, text=True,
                             timeout=10).stdout
    except Exception:
        return None
    pw = re.search(r"SOCKET_POWER:\s*([0-9.]+)\s*W", txt)
    ck = re.search(r"\bCLK:\s*([0-9.]+)\s*MHz", txt)
    if not pw or not ck:
        return None
    return float(pw.group(1)), float(ck.group(1))


def power(args) -> None:
    """Run a command and sample socket power and graphics clock while it runs."""
    import statistics
    import subprocess
    import time
    cmd = args.cmd_args[1:] if args.cmd_args[:1] == ["--"] else args.cmd_args
    child = subprocess.Popen(cmd, stdout=subprocess.PIPE, text=True)
    samples = []
    t0 = time.time()
    while child.poll() is None:
        time.sleep(args.interval)
        s = _smi_sample()
        if s is not None:
            samples.append((time.time() - t0, *s))
    out = child.stdout.read()
    if child.returncode != 0:
        sys.exit(f"command failed with status {child.returncode}")
    if not samples:
        sys.exit("no amd-smi samples")
    top = max(p for _, p, _ in samples)
    loaded = [(t, p, c) for t, p, c in samples if p >= 0.8 * top]
    print("# Socket power and graphics clock while the command runs\n")
    print(f"Command: `python -m kv_cache_eviction_lse_amd.profiling power --interval {args.interval} -- "
          f"{' '.join(cmd)}`\n")
    print(f"Samples: {len(samples)} every {args.interval} s; loaded samples (power >= 80 % of the "
          f"largest): {len(loaded)}\n")
    print("| | socket power W | graphics clock MHz |")
    print("|---|---|---|")
    print(f"| median of loaded samples | {statistics.median(p for _, p, _ in loaded):.0f} | "
          f"{statistics.median(c for _, _, c in loaded):.0f} |")
    print(f"| min / max of loaded samples | {min(p for _, p, _ in loaded):.0f} / "
          f"{max(p for _, p, _ in loaded):.0f} | {min(c for _, _, c in loaded):.0f} / "
          f"{max(c for _, _, c in loaded):.0f} |")
    print("\nCommand output (last line):\n")
    lines = [x for x in out.strip().splitlines() if x.strip()]
    print("```\n" + (lines[-1] if lines else "") + "\n```")


def main() -> None:
    ap = argparse.ArgumentParser()
    sub = ap.add_subparsers(dest="cmd", required=True)
    s = sub.add_parser("stats")
    s.add_argument("--dir", required=True)
    s.add_argument("--command", default="")
    s.add_argument("--all", action="store_true")
    t = sub.add_parser("traffic")
    t.add_argument("--fetch", required=True)
    t.add_argument("--write", required=True)
    t.add_argument("--copy-mib", type=int, required=True)
    t.add_argument("--json", required=True)
    t.add_argument("--algorithmic-bytes", type=float, default=0.0)
    t.add_argument("--command", action="append", default=[])
    t.add_argument("--kernel", default=SCORER, help="kernel name substrings, separated by '|'")
    t.add_argument("--source", default="score.hip", help="csrc file the counters are tied to")
    t.add_argument("--workload", default="llama3_8b_32k")
    cp = sub.add_parser("compute")
    cp.add_argument("--dir", required=True)
    cp.add_argument("--kernel", default=SCORER)
    cp.add_argument("--json", required=True)
    cp.add_argument("--source", default="score.hip")
    cp.add_argument("--workload", default="llama3_8b_32k")
    cp.add_argument("--kernel-us", type=float, default=0.0, help="the kernel's trace time per launch")
    cp.add_argument("--command", action="append", default=[])
    pw = sub.add_parser("power")
    pw.add_argument("--interval", type=float, default=0.5)
    pw.add_argument("cmd_args", nargs=argparse.REMAINDER)
    args = ap.parse_args()
    {"stats": stats, "traffic": traffic, "power": power, "compute": compute}[args.cmd](args)


if __name__ == "__main__":
    main()
