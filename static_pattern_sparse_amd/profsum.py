"""Summarise rocprofv3 output for libfsa kernels (CSV output).

    python -m static_pattern_sparse_amd.profsum <run_kernel_trace.csv>
        per kernel and launch size (grid): dispatches and mean / median / min /
        max duration in microseconds, from the dispatch timestamps.

    python -m static_pattern_sparse_amd.profsum traffic <FETCH_SIZE csv> <WRITE_SIZE csv>
        per kernel and launch size: HBM KiB fetched and written per dispatch,
        each scaled by what the same counter reads for the plain device copy
        in the run (bench.py --calibrate-copy copies 1 GiB: 1 GiB read and
        1 GiB written per copy launch).

    python -m static_pattern_sparse_amd.profsum counters <csv> [<csv> ...]
        per kernel and launch size, from rocprofv3 --pmc runs: the mean L1 ->
        L2 read latency, the L2 hit rate, the bytes the L1 requested from L2
        (staged and read bytes) per token-head, and the texture units' busy
        and stalled fractions (see counter_metrics).
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


# bench.py's launches by kernel and grid: workload name and token-heads per
# launch (B*H*T), so that per-launch counters become per-token-head figures
BENCH_LAUNCHES = {
    ("fwd_mfma_kernel<64>", 4416): ("linear16_bwd_bf16_b8h8t1024d64_w12", 65536),
    ("bwd_dq_mfma_kernel<64>", 4416): ("linear16_bwd_bf16_b8h8t1024d64_w12", 65536),
    ("bwd_dkdv_mfma_kernel<64>", 4736): ("linear16_bwd_bf16_b8h8t1024d64_w12", 65536),
    ("fwd_mfma_kernel<64>", 8768): ("coprime16_bf16_b4h8t4096d64_w6-12", 131072),
    ("bwd_dq_mfma_kernel<64>", 8768): ("coprime16_bf16_b4h8t4096d64_w6-12", 131072),
    ("bwd_dkdv_mfma_kernel<64>", 9376): ("coprime16_bf16_b4h8t4096d64_w6-12", 131072),
}

L2_LINE = 128          # bytes per L1 -> L2 read request (one L2 line)
N_CU = 256
L2_CHANNELS = 128      # 16 per XCD


def _counters(paths):
    agg = collections.defaultdict(lambda: collections.defaultdict(list))
    for path in paths:
        with open(path) as fh:
            for r in csv.DictReader(fh):
                name = kernel_label(r["Kernel_Name"])
                key = (name, int(r["Grid_Size"]) // max(1, int(r["Workgroup_Size"])))
                agg[key][r["Counter_Name"]].append(float(r["Counter_Value"]))
    return {k: {c: sum(v) / len(v) for c, v in d.items()} for k, d in agg.items()}


def counter_metrics(paths):
    """{(kernel, workgroups): metrics} for bench.py's tile-kernel launches:
      l2_read_latency_cycles  TCP_TCC_READ_REQ_LATENCY / TCP_TCC_READ_REQ
      l2_hit_rate             TCC_HIT / (TCC_HIT + TCC_MISS)
      l1_to_l2_bytes_per_token_head  TCP_TCC_READ_REQ x 128 B / token-heads
      td_busy, td_stalled_on_tc      per texture-data unit, as fractions of
                              the kernel's cycles (GRBM_GUI_ACTIVE is summed
                              over the 8 XCDs)
      tcp_pending_stall       TCP_PENDING_STALL_CYCLES per L1, the same
                              fraction (the L1 stalled on misses in flight)
      ta_busy                 TA_BUSY_avr, the same fraction
      l2_tag_stall            TCC_TAG_STALL per L2 channel (16 per XCD), the
                              same fraction
      l2_busy                 TCC_BUSY_avr, the same fraction (a channel with
                              requests in flight)
      l2_req_per_channel_cycle  TCC_REQ per channel per cycle"""
    c = _counters(paths)
    out = {}
    for key, d in c.items():
        if key not in BENCH_LAUNCHES:
            continue
        wl, th = BENCH_LAUNCHES[key]
        m = {"workload": wl}
        if d.get("TCP_TCC_READ_REQ_sum"):
            m["l2_read_latency_cycles"] = d["TCP_TCC_READ_REQ_LATENCY_sum"] / d["TCP_TCC_READ_REQ_sum"]
            m["l1_to_l2_bytes_per_token_head"] = d["TCP_TCC_READ_REQ_sum"] * L2_LINE / th
        if d.get("TCC_HIT_sum") is not None and d.get("TCC_MISS_sum") is not None:
            m["l2_hit_rate"] = d["TCC_HIT_sum"] / max(1.0, d["TCC_HIT_sum"] + d["TCC_MISS_sum"])
        if d.get("GRBM_GUI_ACTIVE") and d.get("TD_TD_BUSY_sum") is not None:
            cyc = d["GRBM_GUI_ACTIVE"] / 8.0
            m["td_busy"] = d["TD_TD_BUSY_sum"] / N_CU / cyc
            m["td_stalled_on_tc"] = d["TD_TC_STALL_sum"] / N_CU / cyc
        if d.get("GRBM_GUI_ACTIVE") and d.get("TCP_PENDING_STALL_CYCLES_sum") is not None:
            m["tcp_pending_stall"] = d["TCP_PENDING_STALL_CYCLES_sum"] / N_CU / (d["GRBM_GUI_ACTIVE"] / 8.0)
        if d.get("GRBM_GUI_ACTIVE") and d.get("TA_BUSY_avr") is not None:
            m["ta_busy"] = d["TA_BUSY_avr"] / (d["GRBM_GUI_ACTIVE"] / 8.0)
        if d.get("GRBM_GUI_ACTIVE") and d.get("TCC_TAG_STALL_sum") is not None:
            m["l2_tag_stall"] = d["TCC_TAG_STALL_sum"] / L2_CHANNELS / (d["GRBM_GUI_ACTIVE"] / 8.0)
        if d.get("GRBM_GUI_ACTIVE") and d.get("TCC_BUSY_avr") is not None:
            m["l2_busy"] = d["TCC_BUSY_avr"] / (d["GRBM_GUI_ACTIVE"] / 8.0)
        if d.get("GRBM_GUI_ACTIVE") and d.get("TCC_REQ_sum") is not None:
            m["l2_req_per_channel_cycle"] = d["TCC_REQ_sum"] / L2_CHANNELS / (d["GRBM_GUI_ACTIVE"] / 8.0)
        out[key] = m
    return out


if __name__ == "__main__":
    if len(sys.argv) > 1 and sys.argv[1] == "counters":
        for (n, wg), m in sorted(counter_metrics(sys.argv[2:]).items()):
            print("%-26s %6d %s" % (n, wg, " ".join(
                f"{k}={v:.3f}" if isinstance(v, float) else f"{k}={v}" for k, v in m.items())))
        sys.exit(0)
    if sys.argv[1] == "traffic":
        res, sf, sw = traffic(sys.argv[2], sys.argv[3])
        print("# copy calibration: FETCH_SIZE x %.4f, WRITE_SIZE x %.4f" % (sf, sw))
        print("%-28s %10s %14s %14s" % ("kernel", "workgroups", "fetch_bytes", "write_bytes"))
        for (n, wg), (fb, wb) in sorted(res.items()):
            line = "%-28s %10d %14.0f %14.0f" % (n, wg, fb, wb)
            if (n, wg) in BENCH_LAUNCHES:
                wl, th = BENCH_LAUNCHES[(n, wg)]
                line += "   %s %.1f B per token-head" % (wl, (fb + wb) / th)
            print(line)
    else:
        print(summarise(sys.argv[1]))
