"""Summaries of rocprofv3 output for profiles/ (measurement tooling).

Reads the CSV files a rocprofv3 run wrote (kernel trace or counter
collection), keeps the dispatches whose full kernel name (template arguments
included) matches --kernel, and prints a markdown table with the command that
produced the data.  Every profiled run launches one product case only (see
bench.py --profile-case), so every dispatch of a kernel in a run belongs to
that case; runs of different cases are given as separate --run arguments.

  python prof_summary.py trace --run LABEL DIR [--run LABEL DIR ...] --cmd CMD ...
  python prof_summary.py pmc --run LABEL DIR ... --cmd CMD ...

`trace` reports dispatch count, average and median duration per kernel.
`pmc` reports the mean of every counter per dispatch per kernel (runs given
the same LABEL, one counter pass each, are merged); with FETCH_SIZE
and WRITE_SIZE present and a device copy of known size in the same runs
(bench.py --profile-case ... copy), it also gives HBM bytes per dispatch scaled
by the counters' reading of that copy.
"""
import argparse
import csv
import glob
import os
import re
import statistics
import sys

ROOT = os.path.dirname(os.path.abspath(__file__))
COPY_KERNEL = "__amd_rocclr_copyBuffer"
COPY_BYTES = 1 << 28  # bench.py --profile-case copy


def short_name(name):
    """'void wq::(anonymous namespace)::gemv_kernel<0, 4, ...>(wq::...)' -> 'gemv_kernel<0, 4, ...>'."""
    n = name.strip().replace("(anonymous namespace)::", "")
    if n.startswith("void "):
        n = n[5:]
    depth = 0
    for i, ch in enumerate(n):  # drop the parameter list after the template arguments
        depth += (ch == "<") - (ch == ">")
        if ch == "(" and depth == 0:
            n = n[:i]
            break
    return re.sub(r"^(?:\w+::)+", "", n)


def rows(dirname, suffix):
    files = sorted(glob.glob(os.path.join(dirname, "**", f"*{suffix}"), recursive=True))
    if not files:
        raise SystemExit(f"no *{suffix} under {dirname}")
    for f in files:
        with open(f, newline="") as fh:
            yield from csv.DictReader(fh)


def col(r, *names):
    for n in names:
        if n in r and r[n] != "":
            return r[n]
    raise KeyError(names[0])


def trace(args):
    out = []
    for label, d in args.run:
        groups = {}
        for r in rows(d, "kernel_trace.csv"):
            name = short_name(col(r, "Kernel_Name"))
            if not re.search(args.kernel, name):
                continue
            grid = int(col(r, "Grid_Size_X", "Grid_Size")) * int(r.get("Grid_Size_Y", 1) or 1)
            dur = (int(col(r, "End_Timestamp")) - int(col(r, "Start_Timestamp"))) / 1e3
            groups.setdefault((name, grid, int(col(r, "Workgroup_Size_X", "Workgroup_Size"))), []).append(dur)
        for (name, grid, wg), ds in sorted(groups.items()):
            out.append((label, name, grid, wg, len(ds), statistics.fmean(ds), statistics.median(ds)))
    print("| case | kernel | grid threads | block | dispatches | avg us | median us |")
    print("|---|---|---|---|---|---|---|")
    for label, name, grid, wg, n, avg, med in out:
        print(f"| {label} | `{name}` | {grid} | {wg} | {n} | {avg:.3f} | {med:.3f} |")


def counters(d, kernel_re):
    """{short kernel name: {counter: [value per dispatch]}} of one run.  Of the
    device copies only the largest-grid ones count (the calibration copy; the
    same kernel also serves the small host-to-device uploads)."""
    per = {}
    copy_grid = max((int(col(r, "Grid_Size")) for r in rows(d, "counter_collection.csv")
                     if short_name(col(r, "Kernel_Name")) == COPY_KERNEL), default=0)
    for r in rows(d, "counter_collection.csv"):
        name = short_name(col(r, "Kernel_Name"))
        if name == COPY_KERNEL:
            if int(col(r, "Grid_Size")) != copy_grid:
                continue
        elif not re.search(kernel_re, name):
            continue
        disp = col(r, "Dispatch_Id", "Correlation_Id")
        per.setdefault(name, {}).setdefault(col(r, "Counter_Name"), {}).setdefault(disp, 0.0)
        # a counter may come as several rows per dispatch (per instance); they add up
        per[name][col(r, "Counter_Name")][disp] += float(col(r, "Counter_Value"))
    return {k: {c: list(v.values()) for c, v in cs.items()} for k, cs in per.items()}


def pmc(args):
    # runs with the same label (one counter pass each, same case) merge into one row per kernel
    merged = {}
    calib = {}
    for label, d in args.run:
        per = counters(d, args.kernel)
        for name, cs in sorted(per.items()):
            if name == COPY_KERNEL:
                for c, vs in cs.items():
                    calib.setdefault(c, []).extend(vs)
                continue
            row = merged.setdefault((label, name), [{}, 0])
            row[0].update({c: statistics.fmean(vs) for c, vs in cs.items()})
            row[1] = max(row[1], max(len(vs) for vs in cs.values()))
    table = [(label, name, cs, n) for (label, name), (cs, n) in merged.items()]
    names = sorted({c for _, _, cs, _ in table for c in cs})
    print("| case | kernel | dispatches | " + " | ".join(names) + " |")
    print("|---|---|---|" + "---|" * len(names))
    for label, name, cs, n in table:
        vals = " | ".join(f"{cs[c]:.6g}" if c in cs else "" for c in names)
        print(f"| {label} | `{name}` | {n} | {vals} |")
    factors = {}
    for c in ("FETCH_SIZE", "WRITE_SIZE"):
        if c in calib:
            kib = statistics.fmean(calib[c])
            factors[c] = kib * 1024 / COPY_BYTES
            print(f"\nCalibration: a device copy of {COPY_BYTES >> 20} MiB reads {c} = {kib:.1f} KiB per "
                  f"dispatch, factor {factors[c]:.4f}.")
    if len(factors) == 2:
        print()
        for label, name, cs, n in table:
            if "FETCH_SIZE" in cs and "WRITE_SIZE" in cs:
                fb = cs["FETCH_SIZE"] * 1024 / factors["FETCH_SIZE"]
                wb = cs["WRITE_SIZE"] * 1024 / factors["WRITE_SIZE"]
                print(f"- {label} `{name}`: hbm_bytes_per_launch: {fb + wb:.0f} (fetch {fb:.0f}, write {wb:.0f})")


def main():
    p = argparse.ArgumentParser()
    p.add_argument("kind", choices=("trace", "pmc"))
    p.add_argument("--run", nargs=2, action="append", metavar=("LABEL", "DIR"), required=True)
    p.add_argument("--kernel", default=r"gemv_kernel|gemm_kernel|ksplit_reduce|gather_x|hadamard",
                   help="regular expression on the short kernel name")
    p.add_argument("--cmd", action="append", default=[], help="command that produced a run (printed)")
    p.add_argument("--title", default="")
    args = p.parse_args()
    if args.title:
        print(f"# {args.title}\n")
    if args.cmd:
        print("Commands (run from the repository root on the GPU box):\n")
        for c in args.cmd:
            print(f"    {c}")
        print()
    sys.path.insert(0, ROOT)
    import bench
    print(f"Kernel sources sha256/16: GEMV {bench.kernel_hash()}, all {bench.kernel_hash(bench.ALL_SOURCES)}\n")
    (trace if args.kind == "trace" else pmc)(args)


if __name__ == "__main__":
    main()
