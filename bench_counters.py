#!/usr/bin/env python3
"""Turn rocprofv3 counter and kernel-trace CSVs of bench.py runs into the
committed summaries under profiles/: `traffic.json`, which bench.py reads
for the `roofline` object's counter figures, and markdown tables.

The counter runs (repository root; one counter group per run, each in a
run of its own):

  python bench.py --profile-cases all --steps 5 > seq.json
  rocprofv3 --pmc FETCH_SIZE -f csv -d D -o f -- python bench.py --profile-cases all --steps 5
  rocprofv3 --pmc WRITE_SIZE -f csv -d D -o w -- python bench.py --profile-cases all --steps 5
  rocprofv3 --pmc SQ_VALU_MFMA_BUSY_CYCLES GRBM_GUI_ACTIVE SQ_INSTS_MFMA -f csv -d D -o b -- \\
      python bench.py --profile-cases all --steps 5
  rocprofv3 --pmc FETCH_SIZE -f csv -d D -o cf -- python bench.py --calibrate-copy
  rocprofv3 --pmc WRITE_SIZE -f csv -d D -o cw -- python bench.py --calibrate-copy

then

  python bench_counters.py counters --seq seq.json --dir D --json profiles/traffic.json \\
      --md profiles/<name>.md

and, for a `rocprofv3 --kernel-trace --stats -f csv -d D -o kt -- python bench.py` run,

  python bench_counters.py stats D/kt_kernel_stats.csv --md profiles/<name>.md --command "..."

How a counter trace is split: `--profile-cases` launches every case once
while setting it up, then a one-element torch fill, then each case
`--steps` times followed by another fill.  The dispatches between two fills
are one case's; the init kernels a stream or K-split plan launches before
its GEMM are counted with the case.  Per call: the counters summed over the
segment divided by `--steps`.

FETCH_SIZE and WRITE_SIZE are in KiB per dispatch; each is scaled by what it
reads for a device-to-device copy of a known size (bench.py
--calibrate-copy: 10 copies of 256 MiB).  MFMA busy = SQ_VALU_MFMA_BUSY_CYCLES
/ (GRBM_GUI_ACTIVE / 8 XCDs x 1024 SIMDs), over the cases' own kernels (the
init kernels excluded).
"""
from __future__ import annotations

import argparse
import csv
import json
import os
import sys

COPY_BYTES = 256 << 20


def read_dispatches(path):
    """[(dispatch id, kernel name, {counter: value})] in dispatch order."""
    disp = {}
    with open(path, newline="") as f:
        for r in csv.DictReader(f):
            d = disp.setdefault(int(r["Dispatch_Id"]), [r["Kernel_Name"], {}])
            c = d[1]
            c[r["Counter_Name"]] = c.get(r["Counter_Name"], 0.0) + float(r["Counter_Value"])
    return [(k, v[0], v[1]) for k, v in sorted(disp.items())]


def find_csv(d, prefix):
    for f in sorted(os.listdir(d)):
        if f.startswith(prefix + "_") and f.endswith("counter_collection.csv"):
            return os.path.join(d, f)
    raise FileNotFoundError(f"no {prefix}_*counter_collection.csv under {d}")


def split_cases(disps, seq):
    """The dispatch segments between the marker fills, one per case (the
    last ncase + 1 fills: the set-up may launch fills of its own)."""
    marks = [i for i, (_, n, _) in enumerate(disps) if seq["marker"] in n]
    ncase = len(seq["profile_cases"])
    if len(marks) < ncase + 1:
        raise SystemExit(f"expected {ncase + 1} marker dispatches, found {len(marks)}")
    marks = marks[-(ncase + 1):]
    segs = []
    for a, b in zip(marks[:-1], marks[1:]):
        seg = disps[a + 1:b]
        for _, n, _ in seg:
            if "baim::" not in n:
                raise SystemExit(f"a dispatch that is not the library's inside a case: {n}")
        segs.append(seg)
    return segs


def calibrate(path, counter):
    vals = [c[counter] for _, n, c in read_dispatches(path) if "copyBuffer" in n and counter in c]
    if not vals:
        raise SystemExit(f"no copy dispatches with {counter} in {path}")
    return COPY_BYTES / 1024 / (sum(vals) / len(vals))


def counters(args):
    with open(args.seq) as f:
        seq = json.loads([ln for ln in f if ln.startswith("{")][-1])
    names, L = seq["profile_cases"], seq["launches"]
    fetch_scale = calibrate(find_csv(args.dir, "cf"), "FETCH_SIZE")
    write_scale = calibrate(find_csv(args.dir, "cw"), "WRITE_SIZE")
    fseg = split_cases(read_dispatches(find_csv(args.dir, "f")), seq)
    wseg = split_cases(read_dispatches(find_csv(args.dir, "w")), seq)
    bseg = split_cases(read_dispatches(find_csv(args.dir, "b")), seq)
    per_case = {}
    for i, name in enumerate(names):
        fk = sum(c.get("FETCH_SIZE", 0.0) for _, _, c in fseg[i]) / L
        wk = sum(c.get("WRITE_SIZE", 0.0) for _, _, c in wseg[i]) / L
        main = [(n, c) for _, n, c in bseg[i] if "init_kernel" not in n]
        busy = sum(c["SQ_VALU_MFMA_BUSY_CYCLES"] for _, c in main)
        active = sum(c["GRBM_GUI_ACTIVE"] for _, c in main) / 8 * 1024
        hbm = fk * 1024 * fetch_scale + wk * 1024 * write_scale
        per_case[name] = {
            "kernel": seq["kernels"][i],
            "fetch_kib_raw": round(fk, 1),
            "write_kib_raw": round(wk, 1),
            "hbm_bytes": int(round(hbm)),
            "algorithmic_bytes": seq["algorithmic_bytes"][i],
            "mfma_busy": round(busy / active, 4) if active else None,
            "mfma_insts": int(round(sum(c["SQ_INSTS_MFMA"] for _, c in main) / L)),
            "dispatches_per_call": len(fseg[i]) / L,
        }
    kernels = {}
    for name in seq["step_cases"]:
        if name not in per_case:
            continue
        pc = per_case[name]
        k = kernels.setdefault(pc["kernel"], {"cases": []})
        k["cases"].append(name)
    for kname, k in kernels.items():
        rows = [per_case[n] for n in k["cases"]]
        n = len(rows)
        k.update({
            "bytes_per_launch": int(sum(r["hbm_bytes"] for r in rows) / n),
            "fetch_bytes_per_launch": int(sum(r["fetch_kib_raw"] * 1024 * fetch_scale for r in rows) / n),
            "write_bytes_per_launch": int(sum(r["write_kib_raw"] * 1024 * write_scale for r in rows) / n),
            "algorithmic_bytes_per_launch": int(sum(r["algorithmic_bytes"] for r in rows) / n),
            "launches_per_step": n,
            "mfma_busy": round(sum(r["mfma_busy"] for r in rows) / n, 4),
        })
    doc = {"kernel_source_sha": seq["kernel_source_sha"], "fetch_scale": round(fetch_scale, 4),
           "write_scale": round(write_scale, 4), "kernels": kernels, "per_case": per_case,
           "source": os.path.relpath(args.md, os.path.dirname(os.path.abspath(__file__)))
           if args.md else None}
    with open(args.json, "w") as f:
        json.dump(doc, f, indent=1)
        f.write("\n")
    if args.md:
        write_counter_md(args.md, doc, seq)


def write_counter_md(path, doc, seq):
    L = seq["launches"]
    out = ["# HBM traffic and MFMA-busy counters: every case bench.py times", "",
           "Commands (repository root; one counter group per run):", "", "```",
           f"python bench.py --profile-cases all --steps {L} > seq.json"]
    for o, pmc in (("f", "FETCH_SIZE"), ("w", "WRITE_SIZE"),
                   ("b", "SQ_VALU_MFMA_BUSY_CYCLES GRBM_GUI_ACTIVE SQ_INSTS_MFMA")):
        out.append(f"timeout -s KILL 120 rocprofv3 --pmc {pmc} -f csv -d D -o {o} -- "
                   f"python bench.py --profile-cases all --steps {L}")
    out += ["timeout -s KILL 60 rocprofv3 --pmc FETCH_SIZE -f csv -d D -o cf -- python bench.py --calibrate-copy",
            "timeout -s KILL 60 rocprofv3 --pmc WRITE_SIZE -f csv -d D -o cw -- python bench.py --calibrate-copy",
            "python bench_counters.py counters --seq seq.json --dir D --json profiles/traffic.json "
            f"--md {path}", "```", "",
            f"Calibration: a 256 MiB device-to-device copy gives FETCH_SIZE x {doc['fetch_scale']} and "
            f"WRITE_SIZE x {doc['write_scale']} = bytes.  FETCH_SIZE counts what leaves the L2 towards "
            "memory (Infinity Cache hits included), so it bounds HBM reads from above.  Per call, "
            f"averaged over {L} back-to-back calls of the case (the init kernel of a stream or "
            "K-split plan counted with it).  MFMA busy = SQ_VALU_MFMA_BUSY_CYCLES / "
            "(GRBM_GUI_ACTIVE / 8 x 1024 SIMDs) over the case's own kernels.", "",
            "| case | kernel | FETCH KiB | WRITE KiB | HBM bytes | algorithmic bytes | ratio | MFMA busy |",
            "|---|---|---|---|---|---|---|---|"]
    for name, r in doc["per_case"].items():
        ratio = r["hbm_bytes"] / r["algorithmic_bytes"] if r["algorithmic_bytes"] else float("nan")
        busy = "-" if r["mfma_busy"] is None else f"{r['mfma_busy']:.3f}"
        out.append(f"| {name} | {r['kernel']} | {r['fetch_kib_raw']:.0f} | {r['write_kib_raw']:.0f} | "
                   f"{r['hbm_bytes'] / 1e6:.1f} MB | {r['algorithmic_bytes'] / 1e6:.1f} MB | "
                   f"{ratio:.2f} | {busy} |")
    out += ["", "Per kernel over the step's cases (what bench.py's `roofline` reads):", ""]
    for k, v in doc["kernels"].items():
        out.append(f"- `{k}` ({', '.join(v['cases'])}): {v['bytes_per_launch'] / 1e6:.1f} MB per launch "
                   f"against {v['algorithmic_bytes_per_launch'] / 1e6:.1f} MB algorithmic; MFMA busy "
                   f"{v['mfma_busy']:.3f}")
    out += ["", f"Kernel sources hash (bench.py uses these figures only while it matches): "
                f"`{doc['kernel_source_sha']}`.", ""]
    with open(path, "w") as f:
        f.write("\n".join(out))


def stats(args):
    rows = []
    with open(args.csv, newline="") as f:
        for r in csv.DictReader(f):
            rows.append(r)
    rows.sort(key=lambda r: -float(r["TotalDurationNs"]))
    out = [f"# {args.title}", "", "Command (repository root):", "", "```", args.command, "```", "",
           "| kernel | calls | total ms | average us | min us | max us | % |",
           "|---|---|---|---|---|---|---|"]
    for r in rows[:args.top]:
        out.append(f"| `{r['Name']}` | {r['Calls']} | {float(r['TotalDurationNs']) / 1e6:.2f} | "
                   f"{float(r['AverageNs']) / 1e3:.1f} | {float(r['MinNs']) / 1e3:.1f} | "
                   f"{float(r['MaxNs']) / 1e3:.1f} | {float(r['Percentage']):.1f} |")
    out.append("")
    with open(args.md, "w") as f:
        f.write("\n".join(out))


def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    sub = ap.add_subparsers(dest="cmd", required=True)
    c = sub.add_parser("counters")
    c.add_argument("--seq", required=True, help="the JSON line of bench.py --profile-cases")
    c.add_argument("--dir", required=True, help="rocprofv3 output folder (f, w, b, cf, cw runs)")
    c.add_argument("--json", required=True)
    c.add_argument("--md", default=None)
    s = sub.add_parser("stats")
    s.add_argument("csv")
    s.add_argument("--md", required=True)
    s.add_argument("--command", required=True)
    s.add_argument("--title", default="Kernel trace")
    s.add_argument("--top", type=int, default=40)
    args = ap.parse_args(argv)
    counters(args) if args.cmd == "counters" else stats(args)


if __name__ == "__main__":
    sys.exit(main())
