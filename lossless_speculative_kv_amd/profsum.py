"""Summaries of rocprofv3 runs of bench.py for profiles/ (measurement tooling).

    python -m lossless_speculative_kv_amd.profsum --workload qwen-32b-layer [--runs gpurun_out]

reads the result databases of the passes below (each run from the repository
root after `cd /tmp && export TMPDIR=/tmp`, with absolute paths), writes
profiles/kernels_<workload>.md, hbm_traffic_<workload>.md and
mfma_<workload>.md, and records the per-launch HBM bytes of the hot-path
kernels in profiles/traffic.json (with the sha256 of each kernel's source,
so bench.py reports them only while the source is unchanged):

    rocprofv3 --kernel-trace --stats -d <runs>/prof_<w> -o run -- python3 -u bench.py <args>
    rocprofv3 --pmc FETCH_SIZE -d <runs>/pmc_fetch_<w> -o run -- python3 -u bench.py <args>
    rocprofv3 --pmc WRITE_SIZE -d <runs>/pmc_write_<w> -o run -- python3 -u bench.py <args>
    rocprofv3 --pmc SQ_VALU_MFMA_BUSY_CYCLES SQ_BUSY_CYCLES SQ_INSTS_VALU_MFMA_MOPS_BF16
              SQ_INSTS_VALU_MFMA_MOPS_F16 GRBM_GUI_ACTIVE -d <runs>/pmc_mfma_<w> -o run -- python3 -u bench.py <args>
    <args> = --workload <w> --steps 3 --warmup 1 --no-cpu-baseline --no-cache-states --quiet --extra none --p1 none --pipeline none

The counters are scaled by a plain device copy of known size (bench.py
--copy-calibration 256, one FETCH_SIZE and one WRITE_SIZE pass into
<runs>/pmc_cfetch and <runs>/pmc_cwrite); without those runs the
calibration stored in traffic.json is used.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import re
import sqlite3
import statistics

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PROFILES = os.path.join(ROOT, "profiles")
BENCH_ARGS = "--steps 3 --warmup 1 --no-cpu-baseline --no-cache-states --quiet --extra none --p1 none --pipeline none"
MFMA_COUNTERS = ("SQ_VALU_MFMA_BUSY_CYCLES SQ_BUSY_CYCLES SQ_INSTS_VALU_MFMA_MOPS_BF16 SQ_INSTS_VALU_MFMA_MOPS_F16 "
                 "GRBM_GUI_ACTIVE")
# hot-path kernels and the source file each is built from
SOURCES = {"draft_kivi_kernel": "draft_attn.hip", "draft_rows_kernel": "draft_attn.hip",
           "verify_kernel": "verify_attn.hip", "verify_merge_kernel": "verify_attn.hip",
           "vocab_stream_kernel": "vocab.hip", "vocab_band_kernel": "vocab.hip", "vocab_ring_kernel": "vocab.hip",
           "vocab_fixup_kernel": "vocab.hip", "vocab_reduce_kernel": "vocab.hip",
           "kivi_quantize_kernel": "round_ops.hip"}
HEADER = ("Run from the repository root on one MI355X (after `cd /tmp && export TMPDIR=/tmp`, with absolute paths to "
          "the repository); summarised by `python -m lossless_speculative_kv_amd.profsum --workload {w}`:\n\n")


def short(name: str) -> str:
    name = re.sub(r"^void ", "", name)
    name = re.sub(r"vc::\(anonymous namespace\)::", "", name)
    name = re.sub(r"\(anonymous namespace\)::", "", name)
    m = re.match(r"([^()]*)\(", name)
    return (m.group(1) if m else name)[:90]


def title(w: str) -> str:
    from .configs import BY_NAME
    c = BY_NAME[w]
    comp = f"KIVI-{c.bits}" if c.kind == "kivi" else ("token drop " + f"{int(100 * c.keep)}%" if c.kind == "tokdrop"
                                                      else c.kind)
    where = ", full cache in pinned host memory" if c.staged else ""
    return (f"{w} round ({comp}, B={c.batch}, {c.n_q_heads} q / {c.n_kv_heads} KV heads, T={c.context}, k={c.k}, "
            f"vocab {c.vocab} x {c.hidden}{where})")


def connect(runs: str, d: str) -> sqlite3.Connection:
    path = os.path.join(runs, d, "run_results.db")
    if not os.path.exists(path):
        raise FileNotFoundError(path)
    return sqlite3.connect(path)


def counters(runs: str, d: str, cname: str) -> dict:
    out: dict = {}
    for kn, v in connect(runs, d).execute("select kernel_name, value from counters_collection where counter_name=?",
                                          (cname,)):
        out.setdefault(short(kn), []).append(v)
    return out


def summarise(w: str, runs: str, out: str = PROFILES) -> None:
    os.makedirs(out, exist_ok=True)
    args = f"--workload {w} {BENCH_ARGS}"
    head = HEADER.format(w=w)
    # ---- kernel trace
    by: dict = {}
    for n, d in connect(runs, f"prof_{w}").execute("select name, duration from kernels"):
        by.setdefault(short(n), []).append(d / 1000.0)
    tot = sum(sum(v) for v in by.values())
    lines = [f"# Kernel trace: {title(w)}\n\n", head,
             f"    rocprofv3 --kernel-trace --stats -d gpurun_out/prof_{w} -o run -- python3 -u bench.py {args}\n\n",
             "Kernel durations in microseconds (setup kernels included):\n\n",
             "| kernel | calls | total us | avg us | median us | min us | max us | % |\n|---|---|---|---|---|---|---|---|\n"]
    for k, v in sorted(by.items(), key=lambda kv: -sum(kv[1])):
        lines.append(f"| `{k}` | {len(v)} | {sum(v):.1f} | {statistics.mean(v):.2f} | {statistics.median(v):.2f} | "
                     f"{min(v):.2f} | {max(v):.2f} | {100 * sum(v) / tot:.2f} |\n")
    with open(os.path.join(out, f"kernels_{w}.md"), "w") as f:
        f.write("".join(lines))
    trace_avg = {k: statistics.mean(v) for k, v in by.items()}

    # ---- HBM traffic
    tpath = os.path.join(out, "traffic.json")
    tsrc = tpath if os.path.exists(tpath) else os.path.join(PROFILES, "traffic.json")
    table = json.load(open(tsrc)) if os.path.exists(tsrc) else {"kernels": {}}
    copy_bytes = 256 * 1024 * 1024
    try:
        cf, cw = counters(runs, "pmc_cfetch", "FETCH_SIZE"), counters(runs, "pmc_cwrite", "WRITE_SIZE")
        ck = max((k for k in cf if "copy" in k.lower()), key=lambda k: statistics.median(cf[k]))
        f_copy, w_copy = statistics.median(cf[ck]), statistics.median(cw[ck])
        cal = {"copy_kernel": ck, "copy_bytes": copy_bytes, "fetch_kib": f_copy, "write_kib": w_copy,
               "fetch_scale": copy_bytes / (f_copy * 1024), "write_scale": copy_bytes / (w_copy * 1024),
               "commands": ["rocprofv3 --pmc FETCH_SIZE -d gpurun_out/pmc_cfetch -o run -- python3 -u bench.py "
                            "--copy-calibration 256",
                            "rocprofv3 --pmc WRITE_SIZE -d gpurun_out/pmc_cwrite -o run -- python3 -u bench.py "
                            "--copy-calibration 256"]}
        table["calibration"] = cal
    except (FileNotFoundError, ValueError):
        cal = table["calibration"]
    fe = counters(runs, f"pmc_fetch_{w}", "FETCH_SIZE")
    wr = counters(runs, f"pmc_write_{w}", "WRITE_SIZE")
    lines = [f"# HBM traffic per launch: {title(w)}\n\n", head,
             f"    rocprofv3 --pmc FETCH_SIZE -d gpurun_out/pmc_fetch_{w} -o run -- python3 -u bench.py {args}\n",
             f"    rocprofv3 --pmc WRITE_SIZE -d gpurun_out/pmc_write_{w} -o run -- python3 -u bench.py {args}\n",
             *[f"    {c}\n" for c in cal["commands"]], "\n",
             f"Calibration: a 256 MiB device copy reads FETCH_SIZE {cal.get('fetch_kib', float('nan')):.1f} KiB and "
             f"WRITE_SIZE {cal.get('write_kib', float('nan')):.1f} KiB per launch, so FETCH_SIZE is scaled by "
             f"{cal['fetch_scale']:.4f} and WRITE_SIZE by {cal['write_scale']:.4f} to give bytes.\n\n",
             "| kernel | launches | FETCH_SIZE KiB (median) | WRITE_SIZE KiB (median) | read bytes | written bytes |\n"
             "|---|---|---|---|---|---|\n"]
    for k in sorted(fe):
        base = k.split("<")[0]
        if base not in SOURCES or k not in wr:
            continue
        fm, wm = statistics.median(fe[k]), statistics.median(wr[k])
        rb, wb = fm * 1024 * cal["fetch_scale"], wm * 1024 * cal["write_scale"]
        lines.append(f"| `{k}` | {len(fe[k])} | {fm:.1f} | {wm:.1f} | {rb / 1e6:.2f} MB | {wb / 1e6:.3f} MB |\n")
        src = "lossless_speculative_kv_amd/csrc/" + SOURCES[base]
        with open(os.path.join(ROOT, src), "rb") as f:
            digest = hashlib.sha256(f.read()).hexdigest()
        table["kernels"][f"{base}@{w}"] = {"kernel": k, "source": src, "source_sha256": digest,
                                           "fetch_bytes": rb, "write_bytes": wb, "launches": len(fe[k])}
    with open(tpath, "w") as f:
        json.dump(table, f, indent=1)
    with open(os.path.join(out, f"hbm_traffic_{w}.md"), "w") as f:
        f.write("".join(lines))

    # ---- MFMA utilisation
    try:
        c = connect(runs, f"pmc_mfma_{w}")
    except FileNotFoundError:
        return
    vals: dict = {}
    for kn, cn, v, disp in c.execute("select kernel_name, counter_name, value, dispatch_id from counters_collection"):
        vals.setdefault(short(kn), {}).setdefault(disp, {}).setdefault(cn, 0.0)
        vals[short(kn)][disp][cn] += v
    lines = [f"# MFMA utilisation: {title(w)}\n\n", head,
             f"    rocprofv3 --pmc {MFMA_COUNTERS} -d gpurun_out/pmc_mfma_{w} -o run -- python3 -u bench.py {args}\n\n",
             "Per launch (medians). MFMA flops = 512 x (MOPS_BF16 + MOPS_F16). Kernel cycles = GRBM_GUI_ACTIVE / 8 (the "
             "counter is summed over the 8 XCDs). MFMA busy = SQ_VALU_MFMA_BUSY_CYCLES / (1024 SIMDs x kernel cycles). "
             "TFLOP/s = issued MFMA flops / the kernel-trace average duration of the same kernel (issued flops include "
             "padding, so they can exceed the algorithmic flops that bench.py reports).\n\n",
             "| kernel | MFMA flops / launch | kernel cycles | MFMA busy | TFLOP/s (trace avg) | % of 2.5 PFLOP/s |\n"
             "|---|---|---|---|---|---|\n"]
    for k in sorted(vals):
        if k.split("<")[0] not in SOURCES:
            continue
        d = list(vals[k].values())
        fl = statistics.median([512 * (x.get("SQ_INSTS_VALU_MFMA_MOPS_BF16", 0) + x.get("SQ_INSTS_VALU_MFMA_MOPS_F16", 0))
                                for x in d])
        if fl == 0:
            continue
        cyc = statistics.median([x.get("GRBM_GUI_ACTIVE", 0) / 8 for x in d])
        busy = statistics.median([x.get("SQ_VALU_MFMA_BUSY_CYCLES", 0) / (1024 * max(1.0, x.get("GRBM_GUI_ACTIVE", 0) / 8))
                                  for x in d])
        t = trace_avg.get(k)
        tf = fl / (t * 1e-6) / 1e12 if t else float("nan")
        lines.append(f"| `{k}` | {fl / 1e9:.2f} G | {cyc:.0f} | {100 * busy:.1f}% | {tf:.0f} | {100 * tf / 2500:.1f}% |\n")
    with open(os.path.join(out, f"mfma_{w}.md"), "w") as f:
        f.write("".join(lines))


def main() -> None:
    ap = argparse.ArgumentParser()
    ap.add_argument("--workload", required=True)
    ap.add_argument("--runs", default=os.path.join(ROOT, "gpurun_out"))
    ap.add_argument("--out", default=PROFILES, help="folder for the summaries and traffic.json (default profiles/)")
    a = ap.parse_args()
    summarise(a.workload, a.runs, a.out)
    print(f"profiles for {a.workload} written")


if __name__ == "__main__":
    main()
