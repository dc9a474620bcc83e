"""Summarise rocprofv3 CSV output of a bench.py run into short markdown files.

Two reports:

  trace    kernel statistics (rocprofv3 --kernel-trace --stats) plus the
           per-arm durations of the sparse FMHA launches;
  traffic  HBM bytes per sparse FMHA launch from two counter runs
           (--pmc FETCH_SIZE, then --pmc WRITE_SIZE), each scaled by what the
           same counter reads for a plain device-to-device copy of known size.

bench.py times its arms in a fixed order (topk 0.4, topk 0.1, dense), each
arm calling the FMHA 2 * (warmup + steps) times (FMHA alone, then block map +
FMHA), and the dense arm 2 + max(5, steps // 2) times; dispatches are assigned
to arms in that order.  The traffic report records the SHA-256 of the FMHA
source so that bench.py stops quoting it once the kernel changes.

A third report, bytes, gives copy-calibrated HBM bytes per dispatch for
every kernel of the library in two counter runs, grouped by kernel and grid.
A fourth, counters, gives the per-arm mean of every counter of one --pmc run
over the sparse FMHA launches (e.g. MfmaUtil, LdsUtil, LDSBankConflict and
SQ_INSTS_VALU_MFMA_MOPS_F16, whose count times 512 is the MFMA flops), next
to the launch's algorithmic flops when the arm's block pairs are given.

Usage:
  python -m block_sparse_attention_sparge_amd.profile_summary trace DIR \
      --steps K --warmup W --command "..." > profiles/x.md
  python -m block_sparse_attention_sparge_amd.profile_summary traffic \
      --fetch DIR --write DIR --copy-fetch DIR --copy-write DIR \
      --copy-bytes N --steps K --warmup W --command "..." > profiles/y.md
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


def arm_slices(steps: int, warmup: int):
    per = 2 * (warmup + steps)
    dense = 2 + max(5, steps // 2)
    return [("topk 0.4", 0, per), ("topk 0.1", per, 2 * per), ("dense", 2 * per, 2 * per + dense)]


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
    out += ["", f"Sparse FMHA launches by bench arm (dispatch order; steps {steps}, warmup {warmup}):", "",
            "| arm | launches | mean us | median us | min us |", "|---|---|---|---|---|"]
    for name, a, b in arm_slices(steps, warmup):
        d = dur[a:b]
        if d:
            out.append(f"| {name} | {len(d)} | {statistics.mean(d):.1f} | {statistics.median(d):.1f} | {min(d):.1f} |")
    return "\n".join(out) + "\n"


def _counter_means(dirpath: str, steps: int, warmup: int):
    rows = list(csv.DictReader(open(_one(dirpath, "*counter_collection.csv"))))
    fm = _fmha_dispatches(rows)
    vals = {}
    for r in fm:
        vals.setdefault(int(r["Dispatch_Id"]), 0.0)
        vals[int(r["Dispatch_Id"])] += float(r["Counter_Value"])
    ordered = [vals[k] for k in sorted(vals)]
    res = {}
    for name, a, b in arm_slices(steps, warmup):
        v = ordered[a:b]
        if v:
            res[name] = sum(v) / len(v)
    return res


def counters_report(dirpath: str, steps: int, warmup: int, command: str, pairs: dict,
                    flops_per_pair: float) -> str:
    rows = list(csv.DictReader(open(_one(dirpath, "*counter_collection.csv"))))
    fm = _fmha_dispatches(rows)
    per = {}
    for r in fm:
        d = per.setdefault(int(r["Dispatch_Id"]), {})
        d[r["Counter_Name"]] = d.get(r["Counter_Name"], 0.0) + float(r["Counter_Value"])
    ids = sorted(per)
    names = sorted({n for d in per.values() for n in d})
    out = ["# Hardware counters of the sparse FMHA (rocprofv3 --pmc)", "", "Command:", "", "```",
           command, "```", "",
           f"Per-arm means over the FMHA launches of the bench (dispatch order; steps {steps}, warmup {warmup}).",
           "", "| arm | launches | " + " | ".join(names) + " |",
           "|---|---|" + "---|" * len(names)]
    extra = []
    for name, a, b in arm_slices(steps, warmup):
        sel = [per[i] for i in ids[a:b]]
        if not sel:
            continue
        means = {n: statistics.fmean(d.get(n, 0.0) for d in sel) for n in names}
        out.append(f"| {name} | {len(sel)} | " + " | ".join(f"{means[n]:.4g}" for n in names) + " |")
        if "SQ_INSTS_VALU_MFMA_MOPS_F16" in means and name in pairs:
            alg = flops_per_pair * pairs[name]
            extra.append(f"- {name}: MFMA flops counted {means['SQ_INSTS_VALU_MFMA_MOPS_F16'] * 512:.4e}, "
                         f"algorithmic {alg:.4e} ({pairs[name]} block pairs x {flops_per_pair:.4g})")
    if extra:
        out += ["", "MFMA work per launch against the algorithmic work:", ""] + extra
    return "\n".join(out) + "\n"


def _copy_kib(dirpath: str) -> float:
    rows = list(csv.DictReader(open(_one(dirpath, "*counter_collection.csv"))))
    per = {}
    for r in rows:
        per.setdefault(int(r["Dispatch_Id"]), 0.0)
        per[int(r["Dispatch_Id"])] += float(r["Counter_Value"])
    vals = list(per.values())
    return statistics.median(vals)


def traffic_report(fetch: str, write: str, copy_fetch: str, copy_write: str, copy_bytes: int,
                   steps: int, warmup: int, command: str) -> str:
    fe = _counter_means(fetch, steps, warmup)
    wr = _counter_means(write, steps, warmup)
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
    for arm in fe:
        b = fe[arm] * fetch_scale * 1024 + wr.get(arm, 0.0) * write_scale * 1024
        summary[arm] = b
        out.append(f"| {arm} | {fe[arm]:.0f} | {wr.get(arm, 0.0):.0f} | {b:.4g} |")
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
    for p in (t,):
        p.add_argument("--steps", type=int, required=True)
        p.add_argument("--warmup", type=int, required=True)
        p.add_argument("--command", required=True)
    f = sub.add_parser("traffic")
    f.add_argument("--fetch", required=True)
    f.add_argument("--write", required=True)
    f.add_argument("--copy-fetch", required=True)
    f.add_argument("--copy-write", required=True)
    f.add_argument("--copy-bytes", type=int, required=True)
    f.add_argument("--steps", type=int, required=True)
    f.add_argument("--warmup", type=int, required=True)
    f.add_argument("--command", required=True)
    c = sub.add_parser("counters")
    c.add_argument("dir")
    c.add_argument("--steps", type=int, required=True)
    c.add_argument("--warmup", type=int, required=True)
    c.add_argument("--command", required=True)
    c.add_argument("--pairs", default="{}", help='JSON {"topk 0.4": pairs, ...}')
    c.add_argument("--flops-per-pair", type=float, default=4.0 * 64 * 64 * 128)
    bt = sub.add_parser("bytes")
    for opt in ("--fetch", "--write", "--copy-fetch", "--copy-write", "--command"):
        bt.add_argument(opt, required=True)
    bt.add_argument("--copy-bytes", type=int, required=True)
    a = ap.parse_args(argv)
    if a.cmd == "trace":
        sys.stdout.write(trace_report(a.dir, a.steps, a.warmup, a.command))
    elif a.cmd == "counters":
        sys.stdout.write(counters_report(a.dir, a.steps, a.warmup, a.command, json.loads(a.pairs),
                                         a.flops_per_pair))
    elif a.cmd == "bytes":
        sys.stdout.write(bytes_report(a.fetch, a.write, a.copy_fetch, a.copy_write, a.copy_bytes, a.command))
    else:
        sys.stdout.write(traffic_report(a.fetch, a.write, a.copy_fetch, a.copy_write, a.copy_bytes,
                                        a.steps, a.warmup, a.command))
    return 0


if __name__ == "__main__":
    sys.exit(main())
