"""Summarise rocprofv3 CSV output of bench.py runs into short markdown files.

Reports:

  trace     kernel statistics (rocprofv3 --kernel-trace --stats) of a default
            bench.py run, plus the durations of the sparse FMHA launches of
            its timed headline region: bench.py runs that region first, so
            they are FMHA dispatches warmup .. warmup + steps - 1;
  traffic   HBM bytes per sparse FMHA launch from two counter runs
            (--pmc FETCH_SIZE, then --pmc WRITE_SIZE) of
            `bench.py --profile-arm ARM`, whose only FMHA launches are that
            arm's; each counter is scaled by what it reads for a plain
            device-to-device copy of known size;
  bytes     copy-calibrated HBM bytes per dispatch for every kernel of the
            library in two counter runs, grouped by kernel and grid;
  counters  the mean of every counter of one --pmc run over the FMHA
            launches of a --profile-arm run (e.g. MfmaUtil, LdsUtil,
            SQ_INSTS_VALU_MFMA_MOPS_F16, whose count times 512 is the MFMA
            flops), next to the launch's algorithmic flops.

In every report the first `--warmup` FMHA dispatches are the untimed warmup
and are left out.  The traffic report records the SHA-256 of the FMHA source
so that bench.py stops quoting it once the kernel changes.

Usage:
  python -m block_sparse_attention_sparge_amd.profile_summary trace DIR \
      --steps K --warmup W --command "..." > profiles/x.md
  python -m block_sparse_attention_sparge_amd.profile_summary traffic \
      --arm "topk 0.4" FETCH_DIR WRITE_DIR [--arm ...] --copy-fetch DIR --copy-write DIR \
      --copy-bytes N --warmup W --command "..." > profiles/y.md
"""
from __future__ import annotations

import argparse
import csv
import glob
import hashlib
import json
import os
import statistics
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
FMHA_SOURCE = os.path.join(PKG, "csrc", "fmha.hip")
FMHA_KERNEL = "fmha_block_kernel"


def source_sha256(path: str = FMHA_SOURCE) -> str:
    with open(path, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()


def _one(dirpath: str, pattern: str) -> str:
    """The most recently written file matching `pattern` under `dirpath`."""
    hits = glob.glob(os.path.join(dirpath, "**", pattern), recursive=True)
    if not hits:
        raise SystemExit(f"no {pattern} under {dirpath}")
    return max(hits, key=os.path.getmtime)


def _fmha_dispatches(rows, key="Dispatch_Id"):
    sel = [r for r in rows if FMHA_KERNEL in r["Kernel_Name"]]
    sel.sort(key=lambda r: int(r[key]))
    return sel


def trace_report(dirpath: str, steps: int, warmup: int, command: str) -> str:
    stats = list(csv.DictReader(open(_one(dirpath, "*kernel_stats.csv"))))
    trace = list(csv.DictReader(open(_one(dirpath, "*kernel_trace.csv"))))
    out = ["# Kernel trace summary (rocprofv3 --kernel-trace --stats)", "",
           "Command:", "", "```", command, "```", "",
           "| kernel | calls | average us | share % |", "|---|---|---|---|"]
    for r in stats:
        name = r["Name"].replace("|", "/")
        if len(name) > 110:
            name = name[:107] + "..."
        out.append(f"| `{name}` | {r['Calls']} | {float(r['AverageNs']) / 1e3:.1f} | {float(r['Percentage']):.2f} |")
    fm = _fmha_dispatches(trace)
    dur = [(int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3 for r in fm]
    d = dur[warmup:warmup + steps]
    out += ["", f"Sparse FMHA launches of the timed headline region (topk 0.4; FMHA dispatches {warmup} .. "
                f"{warmup + steps - 1} of the run):", "",
            "| launches | mean us | median us | min us | max us |", "|---|---|---|---|---|"]
    if d:
        out.append(f"| {len(d)} | {statistics.mean(d):.1f} | {statistics.median(d):.1f} | {min(d):.1f} | "
                   f"{max(d):.1f} |")
    return "\n".join(out) + "\n"


def _counter_mean(dirpath: str, warmup: int) -> float:
    """Mean per FMHA launch (counter values summed over a dispatch's rows)
    after the warmup launches."""
    rows = list(csv.DictReader(open(_one(dirpath, "*counter_collection.csv"))))
    vals = {}
    for r in _fmha_dispatches(rows):
        vals.setdefault(int(r["Dispatch_Id"]), 0.0)
        vals[int(r["Dispatch_Id"])] += float(r["Counter_Value"])
    ordered = [vals[k] for k in sorted(vals)][warmup:]
    if not ordered:
        raise SystemExit(f"no FMHA dispatch after the warmup in {dirpath}")
    return sum(ordered) / len(ordered)


def counters_report(dirpath: str, warmup: int, command: str, arm: str, pairs: int,
                    flops_per_pair: float) -> str:
    rows = list(csv.DictReader(open(_one(dirpath, "*counter_collection.csv"))))
    per = {}
    for r in _fmha_dispatches(rows):
        d = per.setdefault(int(r["Dispatch_Id"]), {})
        d[r["Counter_Name"]] = d.get(r["Counter_Name"], 0.0) + float(r["Counter_Value"])
    sel = [per[i] for i in sorted(per)][warmup:]
    names = sorted({n for d in sel for n in d})
    out = ["# Hardware counters of the sparse FMHA (rocprofv3 --pmc)", "", "Command:", "", "```",
           command, "```", "",
           f"Means over the {len(sel)} FMHA launches of the run after {warmup} warmup launches, arm {arm}.",
           "", "| counter | mean per launch |", "|---|---|"]
    means = {n: statistics.fmean(d.get(n, 0.0) for d in sel) for n in names}
    out += [f"| {n} | {means[n]:.4g} |" for n in names]
    if "SQ_INSTS_VALU_MFMA_MOPS_F16" in means and pairs:
        alg = flops_per_pair * pairs
        out += ["", f"MFMA flops counted {means['SQ_INSTS_VALU_MFMA_MOPS_F16'] * 512:.4e}, algorithmic "
                    f"{alg:.4e} ({pairs} block pairs x {flops_per_pair:.4g})."]
    return "\n".join(out) + "\n"


def _copy_kib(dirpath: str) -> float:
    rows = list(csv.DictReader(open(_one(dirpath, "*counter_collection.csv"))))
    per = {}
    for r in rows:
        per.setdefault(int(r["Dispatch_Id"]), 0.0)
        per[int(r["Dispatch_Id"])] += float(r["Counter_Value"])
    vals = list(per.values())
    return statistics.median(vals)


def traffic_report(arms, copy_fetch: str, copy_write: str, copy_bytes: int, warmup: int,
                   command: str) -> str:
    """arms: list of (arm name, FETCH_SIZE run dir, WRITE_SIZE run dir)."""
    cf, cw = _copy_kib(copy_fetch), _copy_kib(copy_write)
    fetch_scale = copy_bytes / 1024.0 / cf
    write_scale = copy_bytes / 1024.0 / cw
    out = ["# HBM traffic of the sparse FMHA (rocprofv3 --pmc FETCH_SIZE / WRITE_SIZE)", "",
           "Commands:", "", "```", command, "```", "",
           f"Copy calibration: a device-to-device copy of {copy_bytes} bytes reads FETCH_SIZE "
           f"{cf:.0f} KiB and WRITE_SIZE {cw:.0f} KiB per dispatch, so the scale factors are "
           f"{fetch_scale:.3f} (fetch) and {write_scale:.3f} (write).", "",
           "| arm | FETCH_SIZE KiB | WRITE_SIZE KiB | scaled bytes per launch |", "|---|---|---|---|"]
    summary = {}
    for arm, fdir, wdir in arms:
        fe, wr = _counter_mean(fdir, warmup), _counter_mean(wdir, warmup)
        b = fe * fetch_scale * 1024 + wr * write_scale * 1024
        summary[arm] = b
        out.append(f"| {arm} | {fe:.0f} | {wr:.0f} | {b:.4g} |")
    rec = {"kernel": FMHA_KERNEL, "source_sha256": source_sha256(), "fetch_scale": fetch_scale,
           "write_scale": write_scale, "bytes_per_launch": summary}
    out += ["", "Machine-readable line read by bench.py:", "", "traffic_json: " + json.dumps(rec)]
    return "\n".join(out) + "\n"


def read_traffic(path: str, arm: str):
    """Scaled HBM bytes per launch for `arm`, or None when the profile is missing
    or was taken on a different FMHA source."""
    try:
        for line in open(path):
            if line.startswith("traffic_json: "):
                rec = json.loads(line[len("traffic_json: "):])
                if rec.get("source_sha256") != source_sha256():
                    return None
                return rec["bytes_per_launch"].get(arm)
    except OSError:
        return None
    return None


def _short(name: str) -> str:
    """Kernel name without the namespace and argument list."""
    base = name.split("(")[0]
    return base.replace("void ", "").replace("sparge::", "")


def bytes_report(fetch: str, write: str, copy_fetch: str, copy_write: str, copy_bytes: int,
                 command: str) -> str:
    """Copy-calibrated HBM bytes per dispatch for every kernel in the runs,
    grouped by kernel and grid size."""
    cf, cw = _copy_kib(copy_fetch), _copy_kib(copy_write)
    fs, ws = copy_bytes / 1024.0 / cf, copy_bytes / 1024.0 / cw
    groups = {}
    for path, key in ((fetch, "fetch"), (write, "write")):
        for r in csv.DictReader(open(_one(path, "*counter_collection.csv"))):
            if "sparge::" not in r["Kernel_Name"]:
                continue
            g = groups.setdefault((_short(r["Kernel_Name"]), int(r["Grid_Size"])), {"fetch": [], "write": []})
            g[key].append(float(r["Counter_Value"]))
    out = ["# HBM bytes per dispatch of the block-map, combine and decode kernels", "",
           "Commands:", "", "```", command, "```", "",
           f"Copy calibration: a device-to-device copy of {copy_bytes} bytes reads FETCH_SIZE {cf:.0f} KiB and "
           f"WRITE_SIZE {cw:.0f} KiB per dispatch, so the scale factors are {fs:.3f} (fetch) and {ws:.3f} (write).",
           "", "| kernel | grid (threads) | dispatches | read MB | written MB |", "|---|---|---|---|---|"]
    for (name, grid), g in sorted(groups.items()):
        rd = statistics.median(g["fetch"]) * fs * 1024 / 1e6 if g["fetch"] else float("nan")
        wr = statistics.median(g["write"]) * ws * 1024 / 1e6 if g["write"] else float("nan")
        out.append(f"| `{name}` | {grid} | {max(len(g['fetch']), len(g['write']))} | {rd:.2f} | {wr:.2f} |")
    return "\n".join(out) + "\n"


def main(argv=None) -> int:
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    sub = ap.add_subparsers(dest="cmd", required=True)
    t = sub.add_parser("trace")
    t.add_argument("dir")
    t.add_argument("--steps", type=int, required=True)
    t.add_argument("--warmup", type=int, required=True)
    t.add_argument("--command", required=True)
    f = sub.add_parser("traffic")
    f.add_argument("--arm", nargs=3, action="append", required=True, metavar=("NAME", "FETCH_DIR", "WRITE_DIR"))
    f.add_argument("--copy-fetch", required=True)
    f.add_argument("--copy-write", required=True)
    f.add_argument("--copy-bytes", type=int, required=True)
    f.add_argument("--warmup", type=int, required=True)
    f.add_argument("--command", required=True)
    c = sub.add_parser("counters")
    c.add_argument("dir")
    c.add_argument("--warmup", type=int, required=True)
    c.add_argument("--command", required=True)
    c.add_argument("--arm", required=True)
    c.add_argument("--pairs", type=int, default=0)
    c.add_argument("--flops-per-pair", type=float, default=4.0 * 64 * 64 * 128)
    bt = sub.add_parser("bytes")
    for opt in ("--fetch", "--write", "--copy-fetch", "--copy-write", "--command"):
        bt.add_argument(opt, required=True)
    bt.add_argument("--copy-bytes", type=int, required=True)
    a = ap.parse_args(argv)
    if a.cmd == "trace":
        sys.stdout.write(trace_report(a.dir, a.steps, a.warmup, a.command))
    elif a.cmd == "counters":
        sys.stdout.write(counters_report(a.dir, a.warmup, a.command, a.arm, a.pairs, a.flops_per_pair))
    elif a.cmd == "bytes":
        sys.stdout.write(bytes_report(a.fetch, a.write, a.copy_fetch, a.copy_write, a.copy_bytes, a.command))
    else:
        sys.stdout.write(traffic_report(a.arm, a.copy_fetch, a.copy_write, a.copy_bytes, a.warmup, a.command))
    return 0


if __name__ == "__main__":
    sys.exit(main())
