"""Host-side logic of bench.py and the profile summariser (CPU only): the
algorithmic byte counts behind the roofline figures, the check that ties a
committed counter summary to the kernel source it was taken on, the one-GPU
guard, and the kernel labels of the trace summaries."""

from __future__ import annotations

import os
import subprocess
import sys

import bench
from static_pattern_sparse_amd import profsum

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_algorithmic_bytes_per_token_head():
    """Each tensor a kernel must touch, once (D = 64, bf16 inputs, fp32
    outputs): forward q, k, v + out + lse; dq adds dout and Delta; dk/dv reads
    lse and Delta and writes two fp32 rows."""
    sb = bench.stage_bytes(64, 2)
    assert sb == {"fwd": 3 * 128 + 256 + 4, "bwd_dq": 4 * 128 + 4 + 256 + 4,
                  "bwd_dkdv": 4 * 128 + 8 + 512}
    assert sb == {"fwd": 644, "bwd_dq": 776, "bwd_dkdv": 1032}
    assert bench.algo_bytes(64, 2) == {"fwd": 644, "bwd": 4 * 128 + 4 + 768}
    # bf16 out halves the forward's writes; D = 128 doubles the rows
    assert bench.stage_bytes(64, 2, out_bytes=2)["fwd"] == 3 * 128 + 128 + 4
    assert bench.stage_bytes(128, 2)["fwd"] == 3 * 256 + 512 + 4


def test_traffic_summary_follows_the_kernel_source():
    """A committed counter summary counts only while its digest matches the
    current kernel sources."""
    digest = bench.source_digest()
    assert len(digest) == 16
    wl = "linear16_bwd_bf16_b8h8t1024d64_w12"
    for k in ("fwd", "bwd_dq", "bwd_dkdv"):
        path = os.path.join(bench.PROFILES, f"traffic_{k}.txt")
        assert os.path.exists(path), path
        text = open(path).read()
        if f"source_digest: {digest}" in text:
            v = bench.load_traffic(k, 1000, wl)
            assert v is not None and v > 0
        else:
            assert bench.load_traffic(k, 1000, wl) is None
        assert bench.load_traffic(k, 1000, "no_such_workload") is None
    assert bench.load_traffic("no_such_kernel", 1000, wl) is None


def test_consistency_flag():
    """The self-check compares the kernel medians times their launches with
    the host-clock step time and flags a disagreement beyond 10%."""
    per_ms = {"fwd": 0.015, "bwd_dq": 0.022, "bwd_dkdv": 0.023}
    per_step = {"fwd": 16, "bwd_dq": 16, "bwd_dkdv": 16}
    ok = bench.consistency(0.96, per_ms, per_step)
    assert ok["ok"] and abs(ok["sum_kernel_ms"] - 0.96) < 1e-9
    bad = bench.consistency(0.96, dict(per_ms, fwd=0.138), per_step)
    assert not bad["ok"] and bad["ratio"] > 1.1


def test_more_than_one_gpu_is_refused():
    res = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                         capture_output=True, text=True, timeout=120)
    assert res.returncode == 2
    assert "one GPU" in res.stderr


def test_kernel_labels():
    assert profsum.kernel_label("void fsa::(anonymous namespace)::fwd_mfma_kernel<64, float>(...)") \
        == "fwd_mfma_kernel<64>"
    assert profsum.kernel_label("fwd_mfma_kernel<128, unsigned short>(x)").startswith("fwd_mfma_kernel<128,")
    assert profsum.kernel_label("bwd_dkdv_mfma_kernel<64>(a, b)") == "bwd_dkdv_mfma_kernel<64>"
    assert profsum.kernel_label("__amd_rocclr_copyBuffer") == "__amd_rocclr_copyBuffer"
    # the fused-RoPE flag of the tile kernels
    assert profsum.kernel_label("fsa::fwd_mfma_kernel<64, float, false>(x)") == "fwd_mfma_kernel<64>"
    assert profsum.kernel_label("fsa::fwd_mfma_kernel<64, float, true>(x)") == "fwd_mfma_kernel<64,rope>"
    assert profsum.kernel_label("bwd_dq_mfma_kernel<128, false>(a)") == "bwd_dq_mfma_kernel<128>"
    assert profsum.kernel_label("bwd_dkdv_mfma_kernel<64, true>(a)") == "bwd_dkdv_mfma_kernel<64,rope>"


class _FakeHip:
    """Stands in for the HIP runtime: an event is a host timestamp in ms."""

    def __init__(self, ct):
        self.ct = ct

    def hipEventElapsedTime(self, out, e0, e1):
        out._obj.value = e1 - e0
        return 0


def test_event_pairs_time_each_launch_alone():
    """A launch's time runs from the event before it to the event after it;
    the gap from one launch's end to the next launch's start (where the
    records' own cost falls) counts for neither, and the first step is
    dropped."""
    import ctypes
    ev = object.__new__(bench.Events)
    ev.ct, ev.hip = ctypes, _FakeHip(ctypes)
    END = bench.Events.END
    marks, t = [], 0.0
    for step, (a, b) in enumerate(((9.0, 9.0), (1.0, 2.0), (1.5, 2.5), (1.0, 3.0))):
        for name, dur in (("fwd", a), ("bwd", b)):
            marks.append((name, t)); t += dur
            marks.append((END, t)); t += 3.3          # record cost between launches
        marks.append((None, t))
    ev.marks = marks
    med, counts = ev.per_kernel_ms(skip_steps=1)
    assert counts == {"fwd": 3, "bwd": 3}
    assert abs(med["fwd"] - 1.0) < 1e-12 and abs(med["bwd"] - 2.5) < 1e-12


def test_jsonl_records_every_workload(tmp_path):
    """write_jsonl appends one record per workload of the run, each carrying
    the seed root, the main step under the C2+C4 label."""
    import json
    res = {"config": {"workload": "linear16"}, "value": 1.0, "ms_per_step": 2.0,
           "roofline": {"frac": 0.3}, "parity": {"ok": True}, "seed_root": 7,
           "c1": {"workload": "fixed", "value": 3.0}, "t4096": {"workload": "coprime"},
           "t65536": {"workload": "long"}, "decode": {"workload": "dec"}}
    path = tmp_path / "runs.jsonl"
    bench.write_jsonl(str(path), res)
    bench.write_jsonl(str(path), res)
    recs = [json.loads(l) for l in path.read_text().splitlines()]
    assert len(recs) == 10
    labels = [r["record"] for r in recs[:5]]
    assert labels == ["C2+C4 forward+backward", "C1", "C3 forward+backward",
                      "C5 forward+backward, one layer", "decoding step"]
    assert recs[0]["workload"] == "linear16" and recs[0]["roofline"] == {"frac": 0.3}
    assert all(r["seed_root"] == 7 for r in recs)


def test_oracle_baseline_per_slab_matches_per_layer():
    """The per-slab oracle tasks of a long layer give the same parity verdict
    and dalpha as one task per layer (a tiny stack, CPU only)."""
    import types
    import numpy as np
    from static_pattern_sparse_amd import inputs as I
    from oracle import fsa_oracle as O
    B, H, T, D, W, a = 1, 2, 48, 16, 4, 0.7317
    x = I.make_inputs(B, H, T, D, "f32", 77, 0)
    got = {n: np.zeros((B, H, T, D), np.float32) for n in ("out", "dq", "dk", "dv")}
    got["lse"] = np.zeros((B, H, T), np.float32)
    da = 0.0
    for h in range(H):
        sl = [x[n][0, h].astype(np.float64) for n in ("q", "k", "v", "dout")]
        o, l = O.forward_slab(sl[0], sl[1], sl[2], a, W)
        dq, dk, dv, dalpha, _ = O.backward_slab(sl[0], sl[1], sl[2], sl[3], a, W)
        got["out"][0, h], got["lse"][0, h] = o, l
        got["dq"][0, h], got["dk"][0, h], got["dv"][0, h] = dq, dk, dv
        da += dalpha
    wl = types.SimpleNamespace(name="tiny", B=B, H=H, T=T, dtype="f32")
    snap = types.SimpleNamespace(wl=wl, layers=1, W=W, alphas=[a], out_bytes=4,
                                 host=[x], got={0: got}, da={0: da})
    _, p1 = bench.cpu_baseline(snap, passes=1)
    _, p2 = bench.cpu_baseline(snap, passes=1, per_slab=True)
    assert p1["ok"] and p2["ok"]
    assert p1["max_abs"] == p2["max_abs"]
    assert p2["dalpha_rel"] <= 1e-12
