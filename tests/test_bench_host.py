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
    for k in ("fwd", "bwd_dq", "bwd_dkdv"):
        path = os.path.join(bench.PROFILES, f"traffic_{k}.txt")
        assert os.path.exists(path), path
        text = open(path).read()
        if f"source_digest: {digest}" in text:
            v = bench.load_traffic(k, 1000)
            assert v is not None and v > 0
        else:
            assert bench.load_traffic(k, 1000) is None
    assert bench.load_traffic("no_such_kernel", 1000) is None


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
