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
