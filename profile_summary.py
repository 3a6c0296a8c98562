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
import shlex
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


# counters that measure traffic, calibrated against the reference copy: the
# copy reads (R) or writes (W) copy_bytes; FETCH_SIZE / WRITE_SIZE count KiB,
# the TCC_EA0 counters requests
CALIBRATED = {"FETCH_SIZE": "R", "WRITE_SIZE": "W", "TCC_EA0_RDREQ_DRAM_sum": "R", "TCC_EA0_WRREQ_DRAM_sum": "W",
              "TCC_EA0_RDREQ_sum": "R", "TCC_EA0_WRREQ_sum": "W"}


def copy_value(vals, counter: str):
    """The counter's value for one reference copy dispatch (bench.py
    --traffic-probe copies copy_bytes three times after the forward calls;
    the copy kernel also serves the small host-to-device uploads of the
    inputs, so the reference dispatches are the three largest)."""
    for name, cs in vals.items():
        if COPY_KERNEL.search(name) and counter in cs:
            top = sorted(cs[counter], reverse=True)[:3]
            v = statistics.median(top) if top else 0.0
            if v > 0:
                return v
    return None


def copy_factor(vals, counter: str, copy_bytes: int):
    """True bytes per counted KiB-byte (FETCH_SIZE, WRITE_SIZE: copy_bytes /
    (KiB counted per copy * 1024)) and the copy's counted KiB."""
    kib = copy_value(vals, counter)
    return (copy_bytes / (kib * 1024.0), kib) if kib else (None, None)


def counters_cmd(args) -> str:
    vals = counters(args.dirs)
    lines = [f"# {args.title}", "", "commands (repository root, one MI355X, one rocprofv3 --pmc pass each):"]
    lines += [f"  {c}" for c in args.command] + [""]
    fac = {}   # true bytes per counted unit
    for c in CALIBRATED:
        v = copy_value(vals, c)
        if v:
            fac[c] = args.copy_bytes / v
            lines.append(f"calibration: the {args.copy_bytes}-byte device copy "
                         f"({'reads' if CALIBRATED[c] == 'R' else 'writes'} that many bytes) counts {c} {v:.1f} per "
                         f"dispatch -> {fac[c]:.4f} bytes per unit")
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
                extra = f"   ({avg * fac[c] / 1e6:.1f} MB per dispatch, calibrated)"
            lines.append(f"    {c:<36} {avg:>16.1f} per dispatch ({len(v)} dispatches){extra}")
    return "\n".join(lines) + "\n"


def traffic_cmd(args) -> str:
    vf, vw = counters([args.fetch_dir]), counters([args.write_dir])
    ff, fkib = copy_factor(vf, "FETCH_SIZE", args.copy_bytes)
    wf, wkib = copy_factor(vw, "WRITE_SIZE", args.copy_bytes)
    if not ff or not wf:
        raise SystemExit("no reference copy kernel in the counter output")
    # per call: the sum over the matching kernels (a stage may be two
    # launches) of each one's average per dispatch
    def per_call(vals, c):
        ms = [statistics.mean(cs[c]) for n, cs in vals.items() if re.search(args.kernel, n) and cs.get(c)]
        return sum(ms), len(ms), sum(len(cs.get(c, [])) for n, cs in vals.items() if re.search(args.kernel, n))
    fk, nk, nd = per_call(vf, "FETCH_SIZE")
    wk, _, _ = per_call(vw, "WRITE_SIZE")
    if nk == 0:
        raise SystemExit(f"kernel {args.kernel} not in the counter output")
    names = sorted({short(n, 100) for n in vf if re.search(args.kernel, n)})
    fv = [0] * nd
    hbm = fk * 1024 * ff + wk * 1024 * wf
    lines = [f"# {args.title}", "", "commands (repository root, one MI355X, one pass per counter):"]
    lines += [f"  {c}" for c in args.command] + [""]
    lines += [f"kernel: {', '.join(names)}",
              f"calibration: a device copy of {args.copy_bytes} bytes reads FETCH_SIZE {fkib:.1f} KiB and "
              f"WRITE_SIZE {wkib:.1f} KiB per dispatch",
              f"  -> fetch factor {ff:.4f}, write factor {wf:.4f} (bytes per counted byte)",
              "", f"dispatches: {nd} ({nk} kernel(s) per call, summed)",
              f"FETCH_SIZE_KiB_per_dispatch: {fk:.1f}", f"WRITE_SIZE_KiB_per_dispatch: {wk:.1f}",
              f"algorithmic_bytes_per_dispatch: {args.alg_bytes}",
              f"launch_own_bytes_per_dispatch: {args.impl_bytes}",
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
    r.add_argument("--impl-bytes", type=int, default=0)
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
    # the summary's own command, in full (its header lists the rocprofv3 runs)
    own = "python3 profile_summary.py " + " ".join(shlex.quote(a) for a in sys.argv[1:])
    head, _, rest = text.partition("\n\n")
    text = head + "\n\nsummarised by:\n  " + own + "\n\n" + rest
    if args.out:
        with open(args.out, "w") as f:
            f.write(text)
    sys.stdout.write(text)


if __name__ == "__main__":
    main()
