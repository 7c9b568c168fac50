"""Summarise a rocprofv3 kernel trace of libfsa kernels (CSV output).

    python -m static_pattern_sparse_amd.profsum <run_kernel_trace.csv>

Prints, per kernel and launch size (grid), the number of dispatches and the
mean / median / min / max duration in microseconds, from the dispatch start
and end timestamps.
"""

from __future__ import annotations

import collections
import csv
import re
import sys


def summarise(path):
    agg = collections.defaultdict(list)
    with open(path) as fh:
        for r in csv.DictReader(fh):
            m = re.search(r"(\w+_kernel)(<\d+>)?", r["Kernel_Name"])
            name = (m.group(1) + (m.group(2) or "")) if m else r["Kernel_Name"][:40]
            key = (name, int(r["Grid_Size_X"]) // max(1, int(r["Workgroup_Size_X"])))
            agg[key].append((int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3)
    lines = ["%-28s %9s %5s %9s %9s %9s %9s" % ("kernel", "workgroups", "n",
                                                 "mean_us", "median_us", "min_us", "max_us")]
    for (name, wgs), v in sorted(agg.items()):
        v = sorted(v)
        lines.append("%-28s %9d %5d %9.2f %9.2f %9.2f %9.2f" % (
            name, wgs, len(v), sum(v) / len(v), v[len(v) // 2], v[0], v[-1]))
    return "\n".join(lines)


if __name__ == "__main__":
    print(summarise(sys.argv[1]))
