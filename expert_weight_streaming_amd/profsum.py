"""Summaries of rocprofv3 CSV output for this library's kernels.

Reads what `rocprofv3 -f csv -d DIR` wrote (any `*kernel_trace.csv` or
`*counter_collection.csv` below DIR) and prints markdown:

  trace DIR --kernel REGEX [--skip N] [--take M]
      every kernel's calls and mean/min/max duration, then the mean over
      dispatches [N, N+M) of the kernels matching REGEX (in launch order),
      the window a benchmark times;
  counters DIR --kernel REGEX [--skip N] [--take M] [--copy REGEX --copy-bytes B]
      the mean of each counter per dispatch over the same window, in KiB
      where the counter is a size; with --copy, each counter is scaled by
      B / (what it reads for the one dispatch matching the copy REGEX, in
      bytes), so that a counter that sees only part of the traffic still
      gives bytes.

usage: python -m expert_weight_streaming_amd.profsum trace gpurun_out/prof/kt --kernel 'k_stack<' --skip 10 --take 16
"""
import argparse
import csv
import glob
import os
import re
import sys


def _rows(root, suffix):
    files = sorted(glob.glob(os.path.join(root, "**", f"*{suffix}"), recursive=True))
    if not files:
        raise SystemExit(f"no *{suffix} under {root}")
    out = []
    for f in files:
        with open(f, newline="") as fh:
            out.extend(csv.DictReader(fh))
    return out


def _col(row, *names):
    for n in names:
        if n in row:
            return row[n]
    low = {k.lower(): v for k, v in row.items()}
    for n in names:
        if n.lower() in low:
            return low[n.lower()]
    raise KeyError(names)


def _name(row):
    return _col(row, "Kernel_Name", "KernelName", "Kernel-Name")


def _short(name, width=70):
    name = re.sub(r"\(anonymous namespace\)::", "", name)
    return name if len(name) <= width else name[:width - 3] + "..."


def trace(root, kernel, skip, take):
    rows = _rows(root, "kernel_trace.csv")
    disp = []
    for r in rows:
        t0, t1 = int(_col(r, "Start_Timestamp")), int(_col(r, "End_Timestamp"))
        disp.append((t0, _name(r), (t1 - t0) / 1e3))
    disp.sort()
    total = sum(d for _, _, d in disp)
    by = {}
    for _, n, d in disp:
        by.setdefault(n, []).append(d)
    print("| kernel | calls | avg us | min us | max us | % time |")
    print("|---|---:|---:|---:|---:|---:|")
    for n, ds in sorted(by.items(), key=lambda kv: -sum(kv[1])):
        print(f"| `{_short(n)}` | {len(ds)} | {sum(ds) / len(ds):.1f} | {min(ds):.1f} | {max(ds):.1f} | "
              f"{100 * sum(ds) / total:.1f} |")
    pat = re.compile(kernel)
    sel = [(n, d) for _, n, d in disp if pat.search(n)]
    win = sel[skip:skip + take] if take else sel[skip:]
    if not win:
        raise SystemExit(f"no dispatch of {kernel!r} in [{skip}, {skip + take})")
    ds = [d for _, d in win]
    names = sorted({_short(n) for n, _ in win})
    print()
    print(f"Window: dispatches {skip}..{skip + len(ds) - 1} (in launch order) of the {len(sel)} matching "
          f"`{kernel}`: {', '.join(f'`{n}`' for n in names)}")
    print()
    print(f"window_mean_us: {sum(ds) / len(ds):.2f}")
    print(f"window_min_us: {min(ds):.2f}")
    print(f"window_max_us: {max(ds):.2f}")
    print(f"window_dispatches: {len(ds)}")


def counters(root, kernel, skip, take, copy=None, copy_bytes=None):
    rows = _rows(root, "counter_collection.csv")
    per = {}  # dispatch id -> (kernel name, {counter: value})
    for r in rows:
        did = int(_col(r, "Dispatch_Id", "Correlation_Id"))
        n = _name(r)
        c = _col(r, "Counter_Name")
        v = float(_col(r, "Counter_Value"))
        ent = per.setdefault(did, (n, {}))
        ent[1][c] = ent[1].get(c, 0.0) + v
    order = sorted(per)
    pat = re.compile(kernel)
    sel = [per[d] for d in order if pat.search(per[d][0])]
    win = sel[skip:skip + take] if take else sel[skip:]
    if not win:
        raise SystemExit(f"no dispatch of {kernel!r} in [{skip}, {skip + take})")
    names = sorted({c for _, cs in win for c in cs})
    scale = {}
    if copy:
        cp = [per[d] for d in order if re.search(copy, per[d][0])]
        if len(cp) != 1:
            raise SystemExit(f"{len(cp)} dispatches match the copy pattern {copy!r}, want 1")
        for c in names:
            got = cp[0][1].get(c)
            if got:
                scale[c] = copy_bytes / (got * 1024.0)
    kn = sorted({_short(n) for n, _ in win})
    print(f"Window: dispatches {skip}..{skip + len(win) - 1} (in launch order) of the {len(sel)} matching "
          f"`{kernel}`: {', '.join(f'`{n}`' for n in kn)}")
    print()
    print("| counter | mean per dispatch | copy of known size reads | scale | bytes per dispatch |")
    print("|---|---:|---:|---:|---:|")
    for c in names:
        vals = [cs.get(c, 0.0) for _, cs in win]
        m = sum(vals) / len(vals)
        if c in scale:
            cpv = copy_bytes / scale[c] / 1024.0
            print(f"| {c} | {m:.1f} KiB | {cpv:.1f} KiB | {scale[c]:.4f} | {m * 1024.0 * scale[c]:.0f} |")
        else:
            print(f"| {c} | {m:.1f} | | | |")
    print()
    for c in names:
        vals = [cs.get(c, 0.0) for _, cs in win]
        m = sum(vals) / len(vals)
        key = re.sub(r"[^A-Za-z0-9]+", "_", c).strip("_").lower()
        print(f"{key}_mean: {m:.1f}")
        if c in scale:
            print(f"{key}_bytes: {m * 1024.0 * scale[c]:.0f}")


def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("mode", choices=["trace", "counters"])
    ap.add_argument("dir")
    ap.add_argument("--kernel", required=True, help="regular expression on the kernel name")
    ap.add_argument("--skip", type=int, default=0)
    ap.add_argument("--take", type=int, default=0, help="0: all after --skip")
    ap.add_argument("--copy", default=None, help="regular expression naming the calibration copy kernel")
    ap.add_argument("--copy-bytes", type=float, default=float(1 << 30))
    a = ap.parse_args(argv)
    if a.mode == "trace":
        trace(a.dir, a.kernel, a.skip, a.take)
    else:
        counters(a.dir, a.kernel, a.skip, a.take, a.copy, a.copy_bytes)


if __name__ == "__main__":
    sys.exit(main())
