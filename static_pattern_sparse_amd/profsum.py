"""Summarise rocprofv3 output for libfsa kernels (CSV output).

    python -m static_pattern_sparse_amd.profsum <run_kernel_trace.csv>
        per kernel and launch size (grid): dispatches and mean / median / min /
        max duration in microseconds, from the dispatch timestamps.

    python -m static_pattern_sparse_amd.profsum traffic <FETCH_SIZE csv> <WRITE_SIZE csv>
        per kernel and launch size: HBM KiB fetched and written per dispatch,
        each scaled by what the same counter reads for the plain device copy
        in the run (bench.py --calibrate-copy copies 1 GiB: 1 GiB read and
        1 GiB written per copy launch).
"""

from __future__ import annotations

import collections
import csv
import re
import sys


_TYPES = {"unsigned short": "bf16", "float": "f32"}


def kernel_label(full):
    """Short name of a kernel: its name and template arguments, element types
    abbreviated (bf16 bits, f32); the forward's default fp32 output is left
    out, so that fwd_mfma_kernel<64, float> reads fwd_mfma_kernel<64>."""
    m = re.search(r"(\w+_kernel)(?:<([^<>]*)>)?", full)
    if not m:
        return full[:40]
    name, inner = m.group(1), m.group(2)
    if not inner:
        return name
    args = [a.strip() for a in inner.split(",")]
    # the fused-RoPE flag of the tile kernels: dropped when false, "rope" when true
    rope = False
    if args and args[-1] in ("true", "false"):
        rope = args[-1] == "true"
        args = args[:-1]
    if name == "fwd_mfma_kernel" and args and args[-1] == "float":
        args = args[:-1]
    if rope:
        args.append("rope")
    return name + "<" + ",".join(_TYPES.get(a, a) for a in args) + ">"


def summarise(path):
    agg = collections.defaultdict(list)
    with open(path) as fh:
        for r in csv.DictReader(fh):
            name = kernel_label(r["Kernel_Name"])
            key = (name, int(r["Grid_Size_X"]) // max(1, int(r["Workgroup_Size_X"])))
            agg[key].append((int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3)
    lines = ["%-28s %9s %5s %9s %9s %9s %9s" % ("kernel", "workgroups", "n",
                                                 "mean_us", "median_us", "min_us", "max_us")]
    for (name, wgs), v in sorted(agg.items()):
        v = sorted(v)
        lines.append("%-28s %9d %5d %9.2f %9.2f %9.2f %9.2f" % (
            name, wgs, len(v), sum(v) / len(v), v[len(v) // 2], v[0], v[-1]))
    return "\n".join(lines)


COPY_BYTES = 1 << 30


def _counter_means(path):
    agg = collections.defaultdict(list)
    with open(path) as fh:
        for r in csv.DictReader(fh):
            name = kernel_label(r["Kernel_Name"])
            key = (name, int(r["Grid_Size"]) // max(1, int(r["Workgroup_Size"])))
            agg[key].append(float(r["Counter_Value"]))
    return {k: sum(v) / len(v) for k, v in agg.items()}


def traffic(fetch_csv, write_csv):
    """{(kernel, workgroups): (fetch_bytes, write_bytes)} per dispatch, scaled
    by the copy-kernel calibration, plus the two scale factors."""
    f, w = _counter_means(fetch_csv), _counter_means(write_csv)
    cf = [v for (n, _), v in f.items() if "copyBuffer" in n]
    cw = [v for (n, _), v in w.items() if "copyBuffer" in n]
    if not cf or not cw:
        raise SystemExit("no copy kernel in the counter files (run bench.py --calibrate-copy)")
    sf = COPY_BYTES / (cf[0] * 1024.0)
    sw = COPY_BYTES / (cw[0] * 1024.0)
    out = {}
    for key in f:
        if key[0].endswith("_kernel") or "_kernel<" in key[0]:
            if key in w and "copyBuffer" not in key[0]:
                out[key] = (f[key] * 1024.0 * sf, w[key] * 1024.0 * sw)
    return out, sf, sw


if __name__ == "__main__":
    if sys.argv[1] == "traffic":
        res, sf, sw = traffic(sys.argv[2], sys.argv[3])
        print("# copy calibration: FETCH_SIZE x %.4f, WRITE_SIZE x %.4f" % (sf, sw))
        print("%-28s %10s %14s %14s" % ("kernel", "workgroups", "fetch_bytes", "write_bytes"))
        for (n, wg), (fb, wb) in sorted(res.items()):
            print("%-28s %10d %14.0f %14.0f" % (n, wg, fb, wb))
    else:
        print(summarise(sys.argv[1]))
