"""The rocprofv3 summariser behind the committed profiles (CPU only): kernel
trace statistics, HBM traffic scaled by the device copy, and the L1/L2
counter figures, each checked on a small hand-written CSV whose expected
values are worked out in the test."""

from __future__ import annotations

import csv

import pytest

from static_pattern_sparse_amd import profsum

FWD = "void fsa::(anonymous namespace)::fwd_mfma_kernel<64, float, false>(...)"
COPY = "__amd_rocclr_copyBuffer"


def _write(path, fields, rows):
    with open(path, "w", newline="") as fh:
        w = csv.DictWriter(fh, fieldnames=fields)
        w.writeheader()
        for r in rows:
            w.writerow(r)
    return str(path)


def _counter_csv(path, rows):
    """rows: (kernel name, workgroups, counter, value); 64-lane workgroups."""
    return _write(path, ["Kernel_Name", "Grid_Size", "Workgroup_Size", "Counter_Name",
                         "Counter_Value"],
                  [{"Kernel_Name": k, "Grid_Size": 64 * wg, "Workgroup_Size": 64,
                    "Counter_Name": c, "Counter_Value": v} for k, wg, c, v in rows])


def test_trace_statistics(tmp_path):
    """Durations from the dispatch timestamps (ns -> us), grouped by kernel
    and workgroup count: 10, 20 and 60 us give mean 30, median 20."""
    rows = [{"Kernel_Name": FWD, "Grid_Size_X": 64 * 4416, "Workgroup_Size_X": 64,
             "Start_Timestamp": 1000, "End_Timestamp": 1000 + d}
            for d in (10_000, 60_000, 20_000)]
    rows.append({"Kernel_Name": FWD, "Grid_Size_X": 64 * 8768, "Workgroup_Size_X": 64,
                 "Start_Timestamp": 0, "End_Timestamp": 5_000})
    path = _write(tmp_path / "trace.csv", list(rows[0]), rows)
    lines = profsum.summarise(path).splitlines()
    assert lines[0].split()[:3] == ["kernel", "workgroups", "n"]
    by_wg = {int(l.split()[1]): l.split() for l in lines[1:]}
    assert by_wg[4416][0] == "fwd_mfma_kernel<64>"
    assert [float(x) for x in by_wg[4416][2:]] == [3, 30.0, 20.0, 10.0, 60.0]
    assert [float(x) for x in by_wg[8768][2:]] == [1, 5.0, 5.0, 5.0, 5.0]


def test_traffic_is_scaled_by_the_copy(tmp_path):
    """The 1 GiB copy reads and writes 1 GiB. Counters that report half of
    it for reads (512 Ki KiB) and all of it for writes give scales 2 and 1,
    applied to the kernel's KiB per dispatch (mean over dispatches)."""
    fetch = _counter_csv(tmp_path / "f.csv", [
        (COPY, 128, "FETCH_SIZE", 524288.0),
        (FWD, 4416, "FETCH_SIZE", 1000.0), (FWD, 4416, "FETCH_SIZE", 3000.0)])
    write = _counter_csv(tmp_path / "w.csv", [
        (COPY, 128, "WRITE_SIZE", 1048576.0),
        (FWD, 4416, "WRITE_SIZE", 500.0)])
    res, sf, sw = profsum.traffic(fetch, write)
    assert (sf, sw) == (2.0, 1.0)
    assert set(res) == {("fwd_mfma_kernel<64>", 4416)}
    fb, wb = res[("fwd_mfma_kernel<64>", 4416)]
    assert fb == 2000.0 * 1024 * 2.0
    assert wb == 500.0 * 1024 * 1.0


def test_traffic_needs_the_copy(tmp_path):
    f = _counter_csv(tmp_path / "f.csv", [(FWD, 4416, "FETCH_SIZE", 1.0)])
    w = _counter_csv(tmp_path / "w.csv", [(FWD, 4416, "WRITE_SIZE", 1.0)])
    with pytest.raises(SystemExit):
        profsum.traffic(f, w)


def test_counter_metrics(tmp_path):
    """One launch of the headline forward (4416 workgroups, 65536
    token-heads). GRBM_GUI_ACTIVE is summed over the 8 XCDs, so 8000 means
    1000 cycles; per-CU sums divide by 256, per-channel by 128."""
    rows = [
        ("TCP_TCC_READ_REQ_LATENCY_sum", 3_000_000.0),
        ("TCP_TCC_READ_REQ_sum", 10_000.0),
        ("TCC_HIT_sum", 300.0), ("TCC_MISS_sum", 100.0),
        ("GRBM_GUI_ACTIVE", 8000.0),
        ("TD_TD_BUSY_sum", 256 * 500.0), ("TD_TC_STALL_sum", 256 * 100.0),
        ("TCP_PENDING_STALL_CYCLES_sum", 256 * 200.0),
        ("TA_BUSY_avr", 300.0),
        ("TCC_TAG_STALL_sum", 128 * 50.0),
        ("TCC_BUSY_avr", 700.0), ("TCC_REQ_sum", 128 * 250.0),
    ]
    a = _counter_csv(tmp_path / "a.csv", [(FWD, 4416, c, v) for c, v in rows[:5]])
    b = _counter_csv(tmp_path / "b.csv", [(FWD, 4416, c, v) for c, v in rows[4:]]
                     + [(FWD, 1, "TCC_HIT_sum", 1.0)])     # not a bench launch
    m = profsum.counter_metrics([a, b])
    assert set(m) == {("fwd_mfma_kernel<64>", 4416)}
    x = m[("fwd_mfma_kernel<64>", 4416)]
    assert x["workload"] == "linear16_bwd_bf16_b8h8t1024d64_w12"
    assert x["l2_read_latency_cycles"] == 300.0
    assert x["l1_to_l2_bytes_per_token_head"] == 10_000 * 128 / 65536
    assert x["l2_hit_rate"] == 0.75
    assert x["td_busy"] == 0.5 and x["td_stalled_on_tc"] == 0.1
    assert x["tcp_pending_stall"] == 0.2
    assert x["ta_busy"] == 0.3
    assert x["l2_tag_stall"] == 0.05
    assert x["l2_busy"] == 0.7 and x["l2_req_per_channel_cycle"] == 0.25
