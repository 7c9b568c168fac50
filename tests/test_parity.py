"""GPU parity: libfsa (through its C ABI) against the fp64 oracle.

Tolerances (max |GPU - oracle| over every compared element):
  fp32 inputs:  out, lse, dq, dk, dv <= 2e-5
  bf16 inputs:  out, lse, dq, dk, dv <= 2e-3 (inputs are bf16, arithmetic fp32)
  dalpha:       relative error <= 1e-3
Both sides read the same dtype-rounded inputs; the oracle up-casts them exactly
to fp64. Outputs are filled with NaN before each launch so that an element the
kernels fail to write cannot pass.
"""

from __future__ import annotations

import math
import multiprocessing
import os
import sys
from concurrent.futures import ProcessPoolExecutor

import numpy as np
import pytest

from oracle import fsa_oracle as O
from static_pattern_sparse_amd import inputs as I
from tests import _pool

pytestmark = pytest.mark.gpu

TOL = {"f32": 2e-5, "bf16": 2e-3}
DALPHA_RTOL = 1e-3


def _torch():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch


def _say(*a):
    print("[case]", *a, flush=True)
    sys.stdout.flush()


# pattern name -> (oracle base, oracle mode); the library's codes are
# static_pattern_sparse_amd.fsa.PATTERNS
ORACLE_PATTERN = {"fib": ("fib", "lerp"), "fib-round": ("fib", "round"),
                  "pow2": ("pow2", "lerp"), "pow2-round": ("pow2", "round")}


def gpu_forward(x, dtype, alpha, W, pattern="fib"):
    torch = _torch()
    from static_pattern_sparse_amd import fsa as F
    q, k, v = (I.to_device(x[n], dtype) for n in ("q", "k", "v"))
    B, H, T, D = q.shape
    out = torch.full((B, H, T, D), float("nan"), device="cuda")
    lse = torch.full((B, H, T), float("nan"), device="cuda")
    F.fsa_forward(q, k, v, alpha, W, out=out, lse=lse, pattern=F.PATTERNS[pattern])
    torch.cuda.synchronize()
    return out, lse


def gpu_backward(x, dtype, alpha, W, lse, pattern="fib"):
    torch = _torch()
    from static_pattern_sparse_amd import fsa as F
    q, k, v, g = (I.to_device(x[n], dtype) for n in ("q", "k", "v", "dout"))
    B, H, T, D = q.shape
    nan = lambda: torch.full((B, H, T, D), float("nan"), device="cuda")
    dq, dk, dv = nan(), nan(), nan()
    da = torch.full((1,), float("nan"), device="cuda")
    F.fsa_backward(q, k, v, g, lse, alpha, W, dq=dq, dk=dk, dv=dv, dalpha=da,
                   pattern=F.PATTERNS[pattern])
    torch.cuda.synchronize()
    return dq, dk, dv, da


def _np(t):
    return t.detach().cpu().double().numpy()


def _f64(x):
    return {n: a.astype(np.float64) for n, a in x.items()}


def _maxerr(a, b):
    assert np.isfinite(a).all(), "non-finite GPU output"
    return float(np.abs(a - b).max()) if a.size else 0.0


def check_forward(x, dtype, alpha, W, pattern="fib"):
    out, lse = gpu_forward(x, dtype, alpha, W, pattern)
    xd = _f64(x)
    base, mode = ORACLE_PATTERN[pattern]
    ro, rl = O.forward(xd["q"], xd["k"], xd["v"], alpha, W, base=base, mode=mode)
    eo, el = _maxerr(_np(out), ro), _maxerr(_np(lse), rl)
    assert eo <= TOL[dtype], f"out err {eo}"
    assert el <= TOL[dtype], f"lse err {el}"
    return out, lse


def check_backward(x, dtype, alpha, W, lse, pattern="fib"):
    dq, dk, dv, da = gpu_backward(x, dtype, alpha, W, lse, pattern)
    xd = _f64(x)
    base, mode = ORACLE_PATTERN[pattern]
    rq, rk, rv, ra = O.backward(xd["q"], xd["k"], xd["v"], xd["dout"], alpha, W,
                                base=base, mode=mode)
    for name, g, r in (("dq", dq, rq), ("dk", dk, rk), ("dv", dv, rv)):
        e = _maxerr(_np(g), r)
        assert e <= TOL[dtype], f"{name} err {e}"
    a = float(da.item())
    assert abs(a - ra) <= DALPHA_RTOL * abs(ra), f"dalpha {a} vs {ra}"
    return dq, dk, dv, da


def _rand_inputs(B, H, T, D, dtype, seed):
    return I.make_inputs(B, H, T, D, dtype, 90 + seed, 0, rope_base=10000.0)


# ------------------------------------------------------------------ small cases
SMALL = [
    # B, H, T, D, dtype, alpha, W
    (1, 2, 300, 64, "f32", 1.0, 8),
    (2, 1, 1100, 64, "f32", 0.7317, 5),
    (1, 1, 1, 64, "bf16", 1.0, 12),
    (1, 2, 2, 64, "bf16", 0.5, 1),
    (1, 1, 17, 128, "bf16", 1.5, 3),
    (2, 3, 333, 64, "bf16", 0.5666667, 12),
    (1, 2, 1500, 64, "bf16", 1.5, 6),
    (1, 2, 1031, 128, "bf16", 1.2913, 10),
    (1, 2, 250, 64, "bf16", 1.0, 300),          # W > T: causal attention
    (1, 1, 200, 128, "f32", 0.8333333, 12),
    (1, 1, 64, 64, "bf16", 1.0, 1),
    (1, 2, 700, 64, "bf16", 0.6333333, 33),     # three window blocks per tile
    (1, 1, 700, 128, "bf16", 0.6333333, 34),
    (1, 2, 700, 64, "bf16", 0.6333333, 64),     # wide windows: several window pairs
    (2, 1, 500, 128, "bf16", 1.1, 100),
    (1, 2, 300, 64, "bf16", 0.9, 5000),         # W far past T: causal attention
    (2, 1, 29, 64, "bf16", 1.1, 2),
    # B*H a multiple of 8, so that the query-side kernels group heads per XCD:
    # 3 heads per XCD in one group at T1000; 5 heads per XCD at T2050, where
    # half the L2 holds 3 heads' K and V, in a group of 3 and a partial one of 2
    (3, 8, 1000, 64, "bf16", 0.7317, 12),
    (5, 8, 2050, 64, "bf16", 1.2913, 10),
]


@pytest.mark.parametrize("B,H,T,D,dtype,alpha,W", SMALL)
def test_forward_backward_small(B, H, T, D, dtype, alpha, W):
    _say("small", B, H, T, D, dtype, alpha, W)
    alpha = float(np.float32(alpha))
    x = _rand_inputs(B, H, T, D, dtype, T % 7)
    out, lse = check_forward(x, dtype, alpha, W)
    check_backward(x, dtype, alpha, W, lse)


# the power-of-two control base and the rounded (mask) mode: same kernels,
# another tap table
PATTERN_CASES = [
    # B, H, T, D, dtype, alpha, W, pattern
    (1, 2, 600, 64, "bf16", 0.7317, 12, "pow2"),
    (1, 2, 1100, 64, "bf16", 1.0, 8, "pow2"),
    (1, 1, 2100, 64, "bf16", 0.5666667, 12, "pow2"),     # reaches 1024 and 2048
    (1, 2, 500, 64, "bf16", 0.5, 6, "fib-round"),        # ties to even
    (1, 2, 777, 128, "bf16", 1.2913, 10, "fib-round"),
    (1, 1, 1300, 64, "bf16", 0.8333333, 12, "pow2-round"),
    (2, 1, 31, 64, "bf16", 1.5, 3, "pow2-round"),
    (1, 1, 300, 64, "f32", 0.7317, 5, "pow2"),
    (1, 1, 300, 128, "f32", 0.7317, 5, "fib-round"),
    (1, 1, 400, 64, "bf16", 0.7317, 40, "pow2-round"),  # window past the tile kernels
]


@pytest.mark.parametrize("B,H,T,D,dtype,alpha,W,pattern", PATTERN_CASES)
def test_patterns_forward_backward(B, H, T, D, dtype, alpha, W, pattern):
    _say("pattern", pattern, B, H, T, D, dtype, alpha, W)
    alpha = float(np.float32(alpha))
    x = _rand_inputs(B, H, T, D, dtype, T % 5)
    out, lse = check_forward(x, dtype, alpha, W, pattern)
    _, _, _, da = check_backward(x, dtype, alpha, W, lse, pattern)
    if pattern.endswith("round"):
        assert float(da.item()) == 0.0


def test_forward_deterministic_bitwise():
    torch = _torch()
    _say("determinism")
    x = _rand_inputs(2, 2, 700, 64, "bf16", 3)
    o1, l1 = gpu_forward(x, "bf16", 0.7317, 8)
    o2, l2 = gpu_forward(x, "bf16", 0.7317, 8)
    assert torch.equal(o1, o2) and torch.equal(l1, l2)
    g1 = gpu_backward(x, "bf16", 0.7317, 8, l1)
    g2 = gpu_backward(x, "bf16", 0.7317, 8, l1)
    for a, b in zip(g1, g2):
        assert torch.equal(a, b)


def test_split_phase_backward_matches_fused():
    torch = _torch()
    from static_pattern_sparse_amd import fsa as F
    _say("split phase")
    x = _rand_inputs(1, 3, 500, 64, "bf16", 5)
    q, k, v, g = (I.to_device(x[n], "bf16") for n in ("q", "k", "v", "dout"))
    alpha, W = 0.9, 10
    _, lse = F.fsa_forward(q, k, v, alpha, W)
    ref = F.fsa_backward(q, k, v, g, lse, alpha, W)
    ws = torch.empty(F.fsa_backward_workspace_size(1, 3, 500, 64, F.FSA_DTYPE_BF16),
                     dtype=torch.uint8, device="cuda")
    dq, dk, dv = (torch.full_like(ref[0], float("nan")) for _ in range(3))
    da = torch.full((1,), float("nan"), device="cuda")
    F.fsa_backward_dq(q, k, v, g, lse, alpha, W, dq, ws)
    F.fsa_backward_dkdv(q, k, v, g, lse, alpha, W, dk, dv, da, ws)
    torch.cuda.synchronize()
    for a, b in zip((dq, dk, dv, da), ref):
        assert torch.equal(a, b)


def test_integer_offsets_are_pure_gather():
    """alpha = 1 and W >= T reduce to explicit, exactly-indexed attention."""
    _say("integer offsets")
    x = _rand_inputs(1, 2, 1000, 64, "bf16", 4)
    check_forward(x, "bf16", 1.0, 4)
    check_forward(x, "bf16", 1.0, 1000)


@pytest.mark.parametrize("dtype,qscale,alpha,W", [("bf16", 8.0, 0.7317, 12),
                                                  ("bf16", 32.0, 1.2913, 6),
                                                  ("f32", 8.0, 0.8333333, 12)])
def test_sharp_scores(dtype, qscale, alpha, W):
    """q scaled by a power of two (exact in both dtypes): scores of tens of
    units, so the softmax is dominated by a few entries and the running max
    moves often and far (the lazy rescale of the tile kernels and the online
    max of the row-group kernels)."""
    _say("sharp scores", dtype, qscale, alpha, W)
    alpha = float(np.float32(alpha))
    x = _rand_inputs(2, 2, 900, 64, dtype, 40 + int(qscale))
    x["q"] = x["q"] * np.float32(qscale)
    out, lse = gpu_forward(x, dtype, alpha, W)
    dq, dk, dv, da = gpu_backward(x, dtype, alpha, W, lse)
    xd = _f64(x)
    ro, rl = O.forward(xd["q"], xd["k"], xd["v"], alpha, W)
    rq, rk, rv, ra = O.backward(xd["q"], xd["k"], xd["v"], xd["dout"], alpha, W)
    # dk grows with |q| (up to about 80 at q x 32): the max-abs bars, set for
    # outputs of order 1-4, are applied relative to a quarter of each output's
    # largest magnitude when that exceeds 1
    for name, g, r in (("out", out, ro), ("lse", lse, rl), ("dq", dq, rq),
                       ("dk", dk, rk), ("dv", dv, rv)):
        tol = TOL[dtype] * max(1.0, float(np.abs(r).max()) / 4.0)
        e = _maxerr(_np(g), r)
        assert e <= tol, f"{name} err {e} > {tol}"
    a = float(da.item())
    assert abs(a - ra) <= DALPHA_RTOL * abs(ra), f"dalpha {a} vs {ra}"


def test_empty_problem_is_noop():
    torch = _torch()
    from static_pattern_sparse_amd import fsa as F
    _say("empty")
    q = torch.zeros((1, 2, 0, 64), dtype=torch.bfloat16, device="cuda")
    out, lse = F.fsa_forward(q, q, q, 1.0, 8)
    assert out.numel() == 0
    lse_e = torch.zeros((1, 2, 0), device="cuda")
    da = torch.full((1,), float("nan"), device="cuda")
    F.fsa_backward(q, q, q, q, lse_e, 1.0, 8, dalpha=da)
    torch.cuda.synchronize()
    assert float(da.item()) == 0.0


# ------------------------------------------------------------------ workloads
def _alphas(w):
    kind = {"fixed": O.SCHEDULE_FIXED, "linear": O.SCHEDULE_LINEAR,
            "coprime": O.SCHEDULE_COPRIME}[w.schedule]
    return O.schedule(kind, w.layers)


def test_workload_fixed_f32_t256():
    w = I.WORKLOADS["fixed_f32_b1h4t256d64_w8"]
    _say(w.name)
    x = I.workload_inputs(w, 0)
    out, lse = check_forward(x, w.dtype, float(_alphas(w)[0]), 8)
    check_backward(x, w.dtype, float(_alphas(w)[0]), 8, lse)


@pytest.mark.parametrize("layer", [0, 5, 15])
def test_workload_linear16_t1024_fwd_bwd(layer):
    w = I.WORKLOADS["linear16_bwd_bf16_b8h8t1024d64_w12"]
    _say(w.name, layer)
    x = I.workload_inputs(w, layer)
    alpha = float(_alphas(w)[layer])
    out, lse = check_forward(x, w.dtype, alpha, 12)
    check_backward(x, w.dtype, alpha, 12, lse)


@pytest.mark.parametrize("W", [6, 8, 10, 12])
@pytest.mark.parametrize("layer", [1, 10])
def test_workload_coprime16_t4096(layer, W):
    w = I.WORKLOADS["coprime16_bf16_b4h8t4096d64_w6-12"]
    _say(w.name, layer, W)
    x = I.workload_inputs(w, layer, with_dout=(W == 12))
    alpha = float(_alphas(w)[layer])
    out, lse = check_forward(x, w.dtype, alpha, W)
    if W == 12:
        check_backward(x, w.dtype, alpha, W, lse)


@pytest.mark.parametrize("layer", [0, 7, 15])
def test_workload_long_t65536_full(layer):
    """Full-size long-sequence layer (B1 H16 T65536 D128): every element of
    out, lse, dq, dk and dv of all 16 heads against the oracle's forward and
    backward of the same slab, and dalpha against the oracle's sum over the
    heads (heads in parallel spawned processes)."""
    torch = _torch()
    w = I.WORKLOADS["linear16_bf16_b1h16t65536d128_w12"]
    _say(w.name, layer)
    x = I.workload_inputs(w, layer)
    alpha = float(_alphas(w)[layer])
    out, lse = gpu_forward(x, w.dtype, alpha, 12)
    dq, dk, dv, da = gpu_backward(x, w.dtype, alpha, 12, lse)
    got = {n: t[0].float().cpu().numpy() for n, t in
           (("out", out), ("lse", lse), ("dq", dq), ("dk", dk), ("dv", dv))}
    del out, lse, dq, dk, dv
    jobs = [tuple(x[n][0, h] for n in ("q", "k", "v", "dout"))
            + ({n: a[h] for n, a in got.items()}, alpha, 12) for h in range(w.H)]
    # spawned (not forked) workers: they hold no handle of the GPU
    workers = min(16, len(os.sched_getaffinity(0)))
    ctx = multiprocessing.get_context("spawn")
    with ProcessPoolExecutor(max_workers=workers, mp_context=ctx) as ex:
        res = list(ex.map(_pool.slab_check, jobs))
    tol = TOL[w.dtype]
    for h, (errs, _) in enumerate(res):
        for name, e in errs.items():
            assert e <= tol, f"head {h} {name} err {e}"
    ref = math.fsum(r[1] for r in res)
    assert abs(float(da.item()) - ref) <= DALPHA_RTOL * abs(ref)


# ------------------------------------------------------------------ bf16 output
BF16_OUT_CASES = [
    # B, H, T, D, dtype, alpha, W  (bf16: tile kernels; f32: row-group kernels)
    (2, 2, 700, 64, "bf16", 0.7317, 12),
    (1, 2, 333, 128, "bf16", 1.2913, 6),
    (1, 1, 300, 64, "f32", 0.9, 5),
    (1, 1, 260, 64, "bf16", 0.6333333, 40),
]


@pytest.mark.parametrize("B,H,T,D,dtype,alpha,W", BF16_OUT_CASES)
def test_forward_bf16_out(B, H, T, D, dtype, alpha, W):
    """FSA_OUT_BF16: the stored out is the fp32 result rounded to nearest even
    (bit for bit against the fp32 call), lse unchanged; against the oracle the
    bound widens by the rounding, 2^-8 |out|."""
    torch = _torch()
    from static_pattern_sparse_amd import fsa as F
    _say("bf16 out", B, H, T, D, dtype, alpha, W)
    alpha = float(np.float32(alpha))
    x = _rand_inputs(B, H, T, D, dtype, 6)
    q, k, v = (I.to_device(x[n], dtype) for n in ("q", "k", "v"))
    o32, l32 = F.fsa_forward(q, k, v, alpha, W)
    ob = torch.full((B, H, T, D), float("nan"), dtype=torch.bfloat16, device="cuda")
    ob, lb = F.fsa_forward(q, k, v, alpha, W, out=ob)
    torch.cuda.synchronize()
    assert ob.dtype == torch.bfloat16
    assert torch.equal(ob, o32.to(torch.bfloat16))
    assert torch.equal(lb, l32)
    xd = _f64(x)
    ro, _ = O.forward(xd["q"], xd["k"], xd["v"], alpha, W)
    err = np.abs(_np(ob) - ro) - (TOL[dtype] + 2.0 ** -8 * np.abs(ro))
    assert float(err.max()) <= 0.0
