#!/usr/bin/env python3
"""Turn rocprofv3 CSV output into the short text summaries kept in profiles/.

    python profile_summary.py trace DIR --title T --command C [--match RE] [--skip N]
        kernel-trace summary: per kernel, dispatches and average / min / max
        duration (us) from every *kernel_trace.csv under DIR; --skip drops
        each kernel's first N dispatches (warm-up); --match keeps kernels whose
        name matches RE.
    python profile_summary.py counters DIR [DIR ...] --title T --command C [--match RE]
        counter summary: per kernel and counter, the average value per
        dispatch from every *counter_collection.csv under the DIRs (one
        rocprofv3 --pmc pass each); FETCH_SIZE and WRITE_SIZE (KiB) are also
        given in bytes, scaled by what the same counter reads for the
        reference copy kernel of --copy-bytes bytes in the same pass.
    python profile_summary.py traffic FETCH_DIR WRITE_DIR --kernel RE --workload TAG
            --alg-bytes B --source-digest D --title T --command C [--command C2]
        HBM bytes per dispatch of one kernel, calibrated against the copy
        kernel, in the format bench.py reads (hbm_bytes_per_dispatch,
        source_digest).

The summary names the command that produced its input; only committed files
run (bench.py, this file).
"""
from __future__ import annotations

import argparse
import csv
import glob
import os
import re
import statistics
import sys
from collections import defaultdict

COPY_KERNEL = re.compile(r"copyBuffer", re.I)


def _rows(d: str, suffix: str):
    files = sorted(glob.glob(os.path.join(d, "**", f"*{suffix}"), recursive=True))
    if not files:
        raise SystemExit(f"no *{suffix} under {d}")
    for f in files:
        with open(f, newline="") as fh:
            for row in csv.DictReader(fh):
                yield {k.strip().lower(): v for k, v in row.items() if k}


def short(name: str, width: int = 70) -> str:
    name = re.sub(r"^void ", "", name)
    name = name.replace("ssd::(anonymous namespace)::", "").replace("ssd::", "")
    name = name.replace("(anonymous namespace)::", "")
    name = re.sub(r"\(.*$", "", name)
    return name if len(name) <= width else name[:width - 3] + "..."


def trace(args) -> str:
    per = defaultdict(list)
    for r in _rows(args.dir, "kernel_trace.csv"):
        name = r.get("kernel_name", "")
        t0, t1 = int(r.get("start_timestamp", 0)), int(r.get("end_timestamp", 0))
        per[name].append((t0, (t1 - t0) / 1000.0))
    lines = [f"# {args.title}", "", "command (repository root, one MI355X):", f"  {args.command}", ""]
    if args.skip:
        lines.append(f"(each kernel's first {args.skip} dispatches left out: warm-up)")
    lines.append(f"{'kernel':<72}{'calls':>6}{'avg_us':>10}{'min_us':>10}{'max_us':>10}")
    total = 0.0
    for name, v in sorted(per.items(), key=lambda kv: -statistics.mean(d for _, d in kv[1])):
        if args.match and not re.search(args.match, name):
            continue
        d = [x for _, x in sorted(v)][args.skip:]
        if not d:
            continue
        avg = statistics.mean(d)
        total += avg
        lines.append(f"{short(name):<72}{len(d):>6}{avg:>10.2f}{min(d):>10.2f}{max(d):>10.2f}")
    return "\n".join(lines) + "\n"


def counters(dirs, match=None):
    """{kernel: {counter: [values per dispatch]}} and the copy kernel's."""
    vals = defaultdict(lambda: defaultdict(list))
    for d in dirs:
        per_dispatch = defaultdict(lambda: defaultdict(float))
        names = {}
        for r in _rows(d, "counter_collection.csv"):
            key = (d, r.get("dispatch_id", ""))
            names[key] = r.get("kernel_name", "")
            per_dispatch[key][r.get("counter_name", "")] += float(r.get("counter_value", 0) or 0)
        for key, cs in per_dispatch.items():
            for c, v in cs.items():
                vals[names[key]][c].append(v)
    return vals


def copy_factor(vals, counter: str, copy_bytes: int):
    """True bytes per counted byte, from the reference device copy of
    copy_bytes bytes (bench.py --traffic-probe copies it three times after
    the forward calls): copy_bytes / (KiB counted per copy dispatch * 1024).
    The copy kernel also serves the small host-to-device uploads of the
    inputs, so the reference dispatches are the three largest."""
    for name, cs in vals.items():
        if COPY_KERNEL.search(name) and counter in cs:
            top = sorted(cs[counter], reverse=True)[:3]
            kib = statistics.median(top) if top else 0.0
            if kib > 0:
                return copy_bytes / (kib * 1024.0), kib
    return None, None


def counters_cmd(args) -> str:
    vals = counters(args.dirs)
    lines = [f"# {args.title}", "", "commands (repository root, one MI355X, one rocprofv3 --pmc pass each):"]
    lines += [f"  {c}" for c in args.command] + [""]
    fac = {}
    for c in ("FETCH_SIZE", "WRITE_SIZE"):
        f, kib = copy_factor(vals, c, args.copy_bytes)
        if f:
            fac[c] = f
            lines.append(f"calibration: the {args.copy_bytes}-byte device copy reads {c} {kib:.1f} KiB per "
                         f"dispatch -> {f:.4f} true bytes per counted byte")
    lines.append("")
    for name in sorted(vals):
        if args.match and not re.search(args.match, name):
            continue
        if COPY_KERNEL.search(name):
            continue
        lines.append(f"{short(name, 100)}")
        for c in sorted(vals[name]):
            v = vals[name][c]
            avg = statistics.mean(v)
            extra = ""
            if c in fac:
                extra = f"   ({avg * 1024 * fac[c] / 1e6:.1f} MB per dispatch, calibrated)"
            lines.append(f"    {c:<36} {avg:>16.1f} per dispatch ({len(v)} dispatches){extra}")
    return "\n".join(lines) + "\n"


def traffic_cmd(args) -> str:
    vf, vw = counters([args.fetch_dir]), counters([args.write_dir])
    ff, fkib = copy_factor(vf, "FETCH_SIZE", args.copy_bytes)
    wf, wkib = copy_factor(vw, "WRITE_SIZE", args.copy_bytes)
    if not ff or not wf:
        raise SystemExit("no reference copy kernel in the counter output")
    pick = lambda vals, c: [v for n, cs in vals.items() if re.search(args.kernel, n) for v in cs.get(c, [])]
    fv, wv = pick(vf, "FETCH_SIZE"), pick(vw, "WRITE_SIZE")
    if not fv or not wv:
        raise SystemExit(f"kernel {args.kernel} not in the counter output")
    names = sorted({short(n, 100) for n in vf if re.search(args.kernel, n)})
    fk, wk = statistics.mean(fv), statistics.mean(wv)
    hbm = fk * 1024 * ff + wk * 1024 * wf
    lines = [f"# {args.title}", "", "commands (repository root, one MI355X, one pass per counter):"]
    lines += [f"  {c}" for c in args.command] + [""]
    lines += [f"kernel: {', '.join(names)}",
              f"calibration: a device copy of {args.copy_bytes} bytes reads FETCH_SIZE {fkib:.1f} KiB and "
              f"WRITE_SIZE {wkib:.1f} KiB per dispatch",
              f"  -> fetch factor {ff:.4f}, write factor {wf:.4f} (bytes per counted byte)",
              "", f"dispatches: {len(fv)}",
              f"FETCH_SIZE_KiB_per_dispatch: {fk:.1f}", f"WRITE_SIZE_KiB_per_dispatch: {wk:.1f}",
              f"algorithmic_bytes_per_dispatch: {args.alg_bytes}",
              f"hbm_bytes_per_dispatch: {hbm:.0f}",
              f"source_digest: {args.source_digest}"]
    return "\n".join(lines) + "\n"


def main():
    ap = argparse.ArgumentParser()
    sub = ap.add_subparsers(dest="cmd", required=True)
    t = sub.add_parser("trace")
    t.add_argument("dir")
    t.add_argument("--skip", type=int, default=0)
    c = sub.add_parser("counters")
    c.add_argument("dirs", nargs="+")
    c.add_argument("--copy-bytes", type=int, default=256 << 20)
    r = sub.add_parser("traffic")
    r.add_argument("fetch_dir")
    r.add_argument("write_dir")
    r.add_argument("--kernel", required=True)
    r.add_argument("--workload", required=True)
    r.add_argument("--alg-bytes", type=int, required=True)
    r.add_argument("--source-digest", required=True)
    r.add_argument("--copy-bytes", type=int, default=256 << 20)
    for p in (t, c, r):
        p.add_argument("--title", required=True)
        p.add_argument("--command", action="append", required=True)
        p.add_argument("--match", default=None)
        p.add_argument("--out", default=None)
    args = ap.parse_args()
    if args.cmd == "trace":
        args.command = " ; ".join(args.command)
        text = trace(args)
    elif args.cmd == "counters":
        text = counters_cmd(args)
    else:
        text = traffic_cmd(args)
    if args.out:
        with open(args.out, "w") as f:
            f.write(text)
    sys.stdout.write(text)


if __name__ == "__main__":
    main()
