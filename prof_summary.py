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
import shlex
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
            start = int(col(r, "Start_Timestamp"))
            dur = (int(col(r, "End_Timestamp")) - start) / 1e3
            groups.setdefault((name, grid, int(col(r, "Workgroup_Size_X", "Workgroup_Size"))), []).append((start, dur))
        for (name, grid, wg), sd in sorted(groups.items()):
            ds = [dur for _, dur in sorted(sd)][-args.last:] if args.last else [dur for _, dur in sd]
            out.append((label, name, grid, wg, len(ds), statistics.fmean(ds), statistics.median(ds)))
    flops = {k: float(v) for k, v in args.flops}
    byts = args.algorithmic
    print("| case | kernel | grid threads | block | dispatches | avg us | median us | achieved (median) |")
    print("|---|---|---|---|---|---|---|---|")
    totals = {}  # key -> [us, flop]
    for label, name, grid, wg, n, avg, med in out:
        ach = ""
        if label in flops and re.search(args.main_kernel, name):
            ach = f"{flops[label] / med / 1e6:.1f} TFLOP/s ({100 * flops[label] / med / 1e6 / args.mfma_peak:.1f} % of {args.mfma_peak:.0f})"
            m = re.search(args.total_by, label) if args.total_by else None
            t = totals.setdefault(m.group(1) if m else "", [0.0, 0.0])
            t[0] += med
            t[1] += flops[label]
        elif label in byts and re.search(args.main_kernel, name):
            ach = f"{byts[label] / med / 1e3:.1f} GB/s ({100 * byts[label] / med / 1e3 / args.hbm_peak:.1f} % of {args.hbm_peak:.0f})"
        print(f"| {label} | `{name}` | {grid} | {wg} | {n} | {avg:.3f} | {med:.3f} | {ach} |")
    for key, (tot_t, tot_f) in totals.items():
        which = f"Cases matching `{key}`" if key else "Rows with a FLOP count"
        print(f"\n{which} together: {tot_f / 1e9:.1f} GFLOP in {tot_t:.1f} us of median kernel "
              f"time = {tot_f / tot_t / 1e6:.1f} TFLOP/s, {100 * tot_f / tot_t / 1e6 / args.mfma_peak:.1f} % of "
              f"{args.mfma_peak:.0f} TFLOP/s.")


def counters(d, kernel_re, last=0):
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
        disp = int(col(r, "Dispatch_Id", "Correlation_Id"))
        per.setdefault(name, {}).setdefault(col(r, "Counter_Name"), {}).setdefault(disp, 0.0)
        # a counter may come as several rows per dispatch (per instance); they add up
        per[name][col(r, "Counter_Name")][disp] += float(col(r, "Counter_Value"))
    # the last `last` dispatches of each kernel (the measured ones, after the
    # warm-up); every calibration copy
    out = {}
    for k, cs in per.items():
        out[k] = {}
        for c, v in cs.items():
            vals = [v[disp] for disp in sorted(v)]
            out[k][c] = vals[-last:] if last and k != COPY_KERNEL else vals
    return out


def pmc(args):
    # runs with the same label (one counter pass each, same case) merge into one row per kernel
    merged = {}
    calib = {}
    for label, d in args.run:
        per = counters(d, args.kernel, args.last)
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
                alg = args.algorithmic.get(label)
                ratio = f", {(fb + wb) / alg:.4f} x the algorithmic {alg}" if alg else ""
                print(f"- {label} `{name}`: HBM bytes per launch {fb + wb:.0f} (fetch {fb:.0f}, write {wb:.0f}){ratio}")
                if label == args.traffic_of and re.search(args.traffic_kernel, name):
                    traffic = (label, name, fb + wb)
        if args.traffic_of:
            label, name, hbm = traffic
            print(f"\nRoofline traffic of `{name}` ({label}), read by bench.py:\n")
            print(f"- hbm_bytes_per_launch: {hbm:.0f}")
            print(f"- kernel_sources_sha256_16: {__import__('bench').kernel_hash()}")
    # derived per-dispatch figures where the counters are there
    if any("SQ_VALU_MFMA_BUSY_CYCLES" in cs or "SQ_INSTS_VALU" in cs for _, _, cs, _ in table):
        print("\n| case | kernel | VALU instr per wave | MFMA instr per wave | MFMA busy % | VALU busy % (approx) |")
        print("|---|---|---|---|---|---|")
        for label, name, cs, n in table:
            waves = cs.get("SQ_WAVES")
            cyc = cs.get("GRBM_GUI_ACTIVE")
            per_simd = cyc / 8 * 1024 if cyc else None  # 8 XCDs, 1024 SIMDs
            vi = f"{cs['SQ_INSTS_VALU'] / waves:.0f}" if waves and "SQ_INSTS_VALU" in cs else ""
            mi = f"{cs['SQ_INSTS_MFMA'] / waves:.0f}" if waves and "SQ_INSTS_MFMA" in cs else ""
            mb = f"{100 * cs['SQ_VALU_MFMA_BUSY_CYCLES'] / per_simd:.1f}" if per_simd and "SQ_VALU_MFMA_BUSY_CYCLES" in cs else ""
            vb = f"{100 * 4 * cs['SQ_ACTIVE_INST_VALU'] / per_simd:.1f}" if per_simd and "SQ_ACTIVE_INST_VALU" in cs else ""
            print(f"| {label} | `{name}` | {vi} | {mi} | {mb} | {vb} |")


def main():
    p = argparse.ArgumentParser()
    p.add_argument("kind", choices=("trace", "pmc"))
    p.add_argument("--run", nargs=2, action="append", metavar=("LABEL", "DIR"), required=True)
    p.add_argument("--kernel", default=r"gemv_kernel|gemm_kernel|ksplit_reduce|gather_x|hadamard",
                   help="regular expression on the short kernel name")
    p.add_argument("--cmd", action="append", default=[], help="command that produced a run (printed)")
    p.add_argument("--title", default="")
    p.add_argument("--last", type=int, default=0,
                   help="keep only the last N dispatches of each kernel (the measured ones after a warm-up)")
    p.add_argument("--alg", nargs=2, action="append", default=[], metavar=("LABEL", "BYTES"),
                   help="algorithmic bytes per launch of a case (printed beside the counted bytes; trace: "
                        "achieved GB/s of its main kernel)")
    p.add_argument("--flops", nargs=2, action="append", default=[], metavar=("LABEL", "FLOP"),
                   help="FLOP per launch of a case (trace: achieved TFLOP/s of its main kernel)")
    p.add_argument("--main-kernel", default=r"gemv_kernel|gemm_kernel",
                   help="kernel the FLOP / byte counts belong to (regular expression)")
    p.add_argument("--total-by", default="",
                   help="regular expression whose first group on a case label keys the FLOP totals")
    p.add_argument("--hbm-peak", type=float, default=8000.0, help="GB/s")
    p.add_argument("--mfma-peak", type=float, default=2500.0, help="TFLOP/s")
    p.add_argument("--traffic-of", default="", help="label whose HBM bytes bench.py reads as roofline traffic")
    p.add_argument("--traffic-kernel", default="gemv_kernel", help="kernel of that label (regular expression)")
    args = p.parse_args()
    args.algorithmic = {k: int(v) for k, v in args.alg}
    if args.title:
        print(f"# {args.title}\n")
    if args.cmd:
        print("Profiling commands:\n")
        for c in args.cmd:
            print(f"    {c}")
        print()
    own, skip = [], 0
    for a in sys.argv[1:]:  # this summary's own command, without the --cmd / --title texts
        if skip:
            skip -= 1
        elif a in ("--cmd", "--title"):
            skip = 1
        else:
            own.append(a)
    print("Summary command (repository root):\n\n    python prof_summary.py " + shlex.join(own) + "\n")
    sys.path.insert(0, ROOT)
    import bench
    print(f"Kernel sources sha256/16: GEMV {bench.kernel_hash()}, all {bench.kernel_hash(bench.ALL_SOURCES)}\n")
    (trace if args.kind == "trace" else pmc)(args)


if __name__ == "__main__":
    main()
