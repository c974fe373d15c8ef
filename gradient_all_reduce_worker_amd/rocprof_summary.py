"""Summaries of rocprofv3 output for the profiles/ folder.

  python -m gradient_all_reduce_worker_amd.rocprof_summary stats DIR --cmd "..."
      Markdown table from the *_kernel_stats.csv under DIR (per-kernel calls
      and durations).

  python -m gradient_all_reduce_worker_amd.rocprof_summary pmc \
      --fetch DIR1 --write DIR2 --kernel REGEX --probe REGEX \
      --probe-bytes B --alg-bytes A --workload NAME --src FILE --cmd "..."
      HBM bytes per dispatch of the kernels matching REGEX, from a FETCH_SIZE
      run (DIR1) and a WRITE_SIZE run (DIR2). Each counter is scaled by what
      it reads for the probe kernel (a plain copy that reads B bytes and
      writes B bytes), so the result is in bytes whatever the counter's unit.

  python -m gradient_all_reduce_worker_amd.rocprof_summary pmc-table \
      --fetch DIR1 --write DIR2 --probe REGEX --probe-bytes B --cmd "..." \
      NAME=REGEX=ALG_BYTES ...
      The same scaling for several kernels, as a markdown table.

  python -m gradient_all_reduce_worker_amd.rocprof_summary counters \
      --dir DIR [--dir DIR2 ...] --cmd "..." NAME=REGEX=UNITS[=LAUNCHES] ...
      Every counter of the runs (e.g. SQ instruction counts), per call of
      each kernel and per unit of work (UNITS per call).
"""
import argparse
import csv
import glob
import hashlib
import json
import os
import re
import statistics
import subprocess
import sys
from collections import defaultdict


def _rows(pattern_dir: str, suffix: str):
    files = sorted(glob.glob(os.path.join(pattern_dir, "**", f"*{suffix}"), recursive=True))
    if not files:
        raise SystemExit(f"no *{suffix} under {pattern_dir}")
    for f in files:
        with open(f, newline="") as fh:
            for row in csv.DictReader(fh):
                yield {k.strip().lower(): v for k, v in row.items()}


def _short(name: str) -> str:
    try:
        out = subprocess.run(["c++filt"], input=name, capture_output=True, text=True).stdout.strip()
    except OSError:
        out = name
    out = out.replace("(anonymous namespace)::", "")
    # drop the parameter list: the last balanced "(...)" at the end
    if out.endswith(")"):
        depth = 0
        for i in range(len(out) - 1, -1, -1):
            depth += {")": 1, "(": -1}.get(out[i], 0)
            if depth == 0:
                out = out[:i]
                break
    return out.replace("void ", "", 1)[:110]


def cmd_stats(a):
    rows = list(_rows(a.dir, "kernel_stats.csv"))
    rows.sort(key=lambda r: -float(r.get("totaldurationns", 0)))
    print(f"# rocprofv3 kernel statistics: {a.title}\n")
    print(f"Command (run from the repository root on one MI355X):\n\n    {a.cmd}\n")
    print("| kernel | calls | total ms | avg ms | min ms | max ms | % |")
    print("|---|---:|---:|---:|---:|---:|---:|")
    for r in rows:
        ns = float(r["totaldurationns"])
        print(f"| `{_short(r['name'])}` | {r['calls']} | {ns / 1e6:.3f} | "
              f"{float(r['averagens']) / 1e6:.4f} | {float(r['minns']) / 1e6:.4f} | "
              f"{float(r['maxns']) / 1e6:.4f} | {float(r['percentage']):.2f} |")


def _per_kernel(d: str, counter: str):
    vals = defaultdict(list)
    for r in _rows(d, "counter_collection.csv"):
        if r.get("counter_name", "").strip() != counter:
            continue
        vals[r["kernel_name"]].append(float(r["counter_value"]))
    return vals


def cmd_pmc(a):
    fetch = _per_kernel(a.fetch, "FETCH_SIZE")
    write = _per_kernel(a.write, "WRITE_SIZE")
    kre, pre = re.compile(a.kernel), re.compile(a.probe)

    def pick(vals, rx, what):
        hits = {k: v for k, v in vals.items() if rx.search(k)}
        if not hits:
            raise SystemExit(f"no {what} kernel matches {rx.pattern}; kernels: "
                             + ", ".join(sorted(_short(k) for k in vals)))
        return [x for v in hits.values() for x in v]

    pf, pw = pick(fetch, pre, "probe"), pick(write, pre, "probe")
    kf, kw = pick(fetch, kre, "target"), pick(write, kre, "target")
    # the probe is the largest dispatch of its kernel name (the 1 GiB copy)
    f_scale = a.probe_bytes / max(pf)
    w_scale = a.probe_bytes / max(pw)
    fb = statistics.mean(kf) * f_scale
    wb = statistics.mean(kw) * w_scale
    with open(a.src, "rb") as fh:
        src_hash = hashlib.sha256(fh.read()).hexdigest()[:16]
    out = {
        "workload": a.workload, "kernel_regex": a.kernel, "command": a.cmd,
        "dispatches": {"fetch_run": len(kf), "write_run": len(kw)},
        "probe": {"regex": a.probe, "bytes_each_way": a.probe_bytes,
                  "fetch_counter": max(pf), "write_counter": max(pw)},
        "fetch_bytes_per_launch": fb, "write_bytes_per_launch": wb,
        "hbm_bytes_per_launch": fb + wb, "alg_bytes_per_launch": a.alg_bytes,
        "traffic_over_alg": (fb + wb) / a.alg_bytes if a.alg_bytes else None,
        "ring_src_sha256_16": src_hash,
    }
    json.dump(out, sys.stdout, indent=1)
    print()


def cmd_pmc_table(a):
    """Markdown table: per kernel, scaled fetch/write bytes per call against
    the algorithmic bytes given as NAME=REGEX=BYTES[=LAUNCHES] (LAUNCHES: a
    call that runs as several launches of the kernel; default 1)."""
    fetch = _per_kernel(a.fetch, "FETCH_SIZE")
    write = _per_kernel(a.write, "WRITE_SIZE")
    pre = re.compile(a.probe)
    pf = max(x for k, v in fetch.items() if pre.search(k) for x in v)
    pw = max(x for k, v in write.items() if pre.search(k) for x in v)
    print(f"# HBM traffic per call from rocprofv3 PMC counters: {a.title}\n")
    print("FETCH_SIZE and WRITE_SIZE were collected in two separate runs and scaled by what")
    print(f"each reads for a plain copy of {a.probe_bytes:.0f} bytes each way (`{a.probe}`:")
    print(f"FETCH_SIZE {pf:.2f}, WRITE_SIZE {pw:.2f}).\n")
    print(f"Commands (run from the repository root on one MI355X):\n\n    {a.cmd}\n")
    print("| kernel | launches | read GB | written GB | algorithmic GB | traffic / algorithmic |")
    print("|---|---:|---:|---:|---:|---:|")
    for spec in a.kernels:
        parts = spec.split("=")
        name, rx, alg = parts[:3]
        per_call = int(parts[3]) if len(parts) > 3 else 1
        r = re.compile(rx)
        kf = [x for k, v in fetch.items() if r.search(k) for x in v]
        kw = [x for k, v in write.items() if r.search(k) for x in v]
        fb = statistics.mean(kf) * a.probe_bytes / pf * per_call
        wb = statistics.mean(kw) * a.probe_bytes / pw * per_call
        print(f"| `{name}` | {len(kf)} | {fb / 1e9:.3f} | {wb / 1e9:.3f} | {float(alg) / 1e9:.3f} | "
              f"{(fb + wb) / float(alg):.4f} |")


def cmd_counters(a):
    """Markdown table: per kernel, every counter of the runs under DIRs,
    summed over a call's launches and averaged over calls, and divided by
    the call's units (NAME=REGEX=UNITS[=LAUNCHES]: e.g. UNITS = coordinates
    a call processes, LAUNCHES = launches per call, default 1)."""
    per = defaultdict(lambda: defaultdict(float))      # (kernel, dispatch) -> counter -> value
    names = {}
    for d in a.dir:
        for r in _rows(d, "counter_collection.csv"):
            key = (d, r["kernel_name"], r.get("dispatch_id", r.get("correlation_id", "")))
            per[key][r["counter_name"].strip()] += float(r["counter_value"])
            names[r["counter_name"].strip()] = True
    counters = sorted(names)
    print(f"# rocprofv3 counters per call: {a.title}\n")
    print(f"Commands (run from the repository root on one MI355X):\n\n    {a.cmd}\n")
    print("Each counter is summed over a call's launches and averaged over the calls; "
          "the second figure divides it by the units the call processes.\n")
    print("| kernel | units per call | " + " | ".join(counters) + " |")
    print("|---|---:|" + "---:|" * len(counters))
    for spec in a.kernels:
        parts = spec.split("=")
        name, rx, units = parts[0], re.compile(parts[1]), float(parts[2])
        per_call = int(parts[3]) if len(parts) > 3 else 1
        cells = []
        for c in counters:
            vals = [v[c] for (d, k, _), v in per.items() if rx.search(k) and c in v]
            if not vals:
                cells.append("—")
                continue
            call = sum(vals) / (len(vals) / per_call)
            cells.append(f"{call:.4g} ({call / units:.3g})")
        print(f"| `{name}` | {units:.4g} | " + " | ".join(cells) + " |")


def main():
    ap = argparse.ArgumentParser()
    sub = ap.add_subparsers(dest="mode", required=True)
    s = sub.add_parser("stats")
    s.add_argument("dir")
    s.add_argument("--cmd", required=True)
    s.add_argument("--title", default="")
    p = sub.add_parser("pmc")
    p.add_argument("--fetch", required=True)
    p.add_argument("--write", required=True)
    p.add_argument("--kernel", required=True)
    p.add_argument("--probe", required=True)
    p.add_argument("--probe-bytes", type=float, required=True)
    p.add_argument("--alg-bytes", type=float, required=True)
    p.add_argument("--workload", required=True)
    p.add_argument("--src", required=True)
    p.add_argument("--cmd", required=True)
    t = sub.add_parser("pmc-table")
    t.add_argument("--fetch", required=True)
    t.add_argument("--write", required=True)
    t.add_argument("--probe", required=True)
    t.add_argument("--probe-bytes", type=float, required=True)
    t.add_argument("--title", default="")
    t.add_argument("--cmd", required=True)
    t.add_argument("kernels", nargs="+", help="NAME=REGEX=ALG_BYTES")
    c = sub.add_parser("counters")
    c.add_argument("--dir", action="append", required=True)
    c.add_argument("--title", default="")
    c.add_argument("--cmd", required=True)
    c.add_argument("kernels", nargs="+", help="NAME=REGEX=UNITS[=LAUNCHES]")
    a = ap.parse_args()
    {"stats": cmd_stats, "pmc": cmd_pmc, "pmc-table": cmd_pmc_table,
     "counters": cmd_counters}[a.mode](a)


if __name__ == "__main__":
    main()
