"""GPU parity of the decoding step (fsa_decode, through the C ABI) against the
fp64 oracle's decode.

Tolerances as for the sequence kernels: max |GPU - oracle| <= 2e-5 (fp32
inputs) and 2e-3 (bf16 inputs) on out and lse. Outputs are filled with NaN
before each launch so that an element the kernel fails to write cannot pass.
"""

from __future__ import annotations

import sys

import numpy as np
import pytest

from oracle import fsa_oracle as O
from static_pattern_sparse_amd import inputs as I

pytestmark = pytest.mark.gpu

TOL = {"f32": 2e-5, "bf16": 2e-3}
ORACLE_PATTERN = {"fib": ("fib", "lerp"), "fib-round": ("fib", "round"),
                  "pow2": ("pow2", "lerp"), "pow2-round": ("pow2", "round")}


def _torch():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch


def _say(*a):
    print("[case]", *a, flush=True)
    sys.stdout.flush()


def gpu_decode(x, dtype, alpha, W, pattern="fib", k=None, v=None):
    torch = _torch()
    from static_pattern_sparse_amd import fsa as F
    q = I.to_device(x["q"], dtype)
    k = I.to_device(x["k"], dtype) if k is None else k
    v = I.to_device(x["v"], dtype) if v is None else v
    pos = torch.from_numpy(np.asarray(x["pos"], dtype=np.int32)).to("cuda")
    B, H, D = q.shape
    out = torch.full((B, H, D), float("nan"), device="cuda")
    lse = torch.full((B, H), float("nan"), device="cuda")
    F.fsa_decode(q, k, v, pos, alpha, W, out=out, lse=lse, pattern=F.PATTERNS[pattern])
    torch.cuda.synchronize()
    return out.cpu().double().numpy(), lse.cpu().double().numpy()


def _f64(x):
    return {n: (a.astype(np.float64) if n != "pos" else a) for n, a in x.items()}


def check_decode(x, dtype, alpha, W, pattern="fib"):
    out, lse = gpu_decode(x, dtype, alpha, W, pattern)
    xd = _f64(x)
    base, mode = ORACLE_PATTERN[pattern]
    ro, rl = O.decode(xd["q"], xd["k"], xd["v"], xd["pos"], alpha, W, base=base, mode=mode)
    assert np.isfinite(out).all() and np.isfinite(lse).all()
    eo, el = float(np.abs(out - ro).max()), float(np.abs(lse - rl).max())
    assert eo <= TOL[dtype], f"out err {eo}"
    assert el <= TOL[dtype], f"lse err {el}"
    return out, lse


CASES = [
    # B, H, T_cap, D, dtype, alpha, W, pattern, positions
    (5, 3, 2100, 64, "bf16", 0.5666667, 12, "fib", [0, 1, 11, 1500, 2099]),
    (4, 2, 1300, 128, "bf16", 1.2913, 10, "pow2", [5, 600, 1299, 63]),
    (3, 2, 900, 64, "f32", 0.7317, 5, "fib-round", [899, 4, 377]),
    (2, 2, 1100, 128, "f32", 0.5, 6, "pow2-round", [1099, 512]),
    (2, 1, 3000, 64, "bf16", 1.0, 5000, "fib", [2999, 100]),   # W > T: causal
    (1, 1, 17, 64, "bf16", 1.5, 1, "fib", [16]),
    (6, 1, 4096, 64, "bf16", 1.5, 12, "fib", [4095, 1480, 1481, 1482, 987, 2047]),
]


@pytest.mark.parametrize("B,H,T,D,dtype,alpha,W,pattern,positions", CASES)
def test_decode_small(B, H, T, D, dtype, alpha, W, pattern, positions):
    _say("decode", B, H, T, D, dtype, alpha, W, pattern, positions)
    alpha = float(np.float32(alpha))
    x = I.make_decode_inputs(B, H, T, D, dtype, 70 + T % 11, 0, positions)
    check_decode(x, dtype, alpha, W, pattern)


def test_decode_reads_no_row_past_its_position():
    """Cache rows after each query's position hold NaN: the outputs stay
    finite and equal to the run on the clean cache, bit for bit."""
    torch = _torch()
    _say("decode NaN past position")
    pos = [700, 33, 1023]
    x = I.make_decode_inputs(3, 2, 1024, 64, "bf16", 81, 0, pos)
    ref = gpu_decode(x, "bf16", 0.8333333, 12)
    k = I.to_device(x["k"], "bf16")
    v = I.to_device(x["v"], "bf16")
    for b, i in enumerate(pos):
        k[b, :, i + 1:] = float("nan")
        v[b, :, i + 1:] = float("nan")
    got = gpu_decode(x, "bf16", 0.8333333, 12, k=k, v=v)
    assert np.isfinite(got[0]).all()
    assert np.array_equal(got[0], ref[0]) and np.array_equal(got[1], ref[1])


def test_decode_bad_position_writes_nan():
    _say("decode bad position")
    x = I.make_decode_inputs(3, 2, 300, 64, "bf16", 82, 0, [299, 0, 10])
    x["pos"] = np.array([299, -1, 300], dtype=np.int32)
    out, lse = gpu_decode(x, "bf16", 1.0, 8)
    assert np.isnan(out[1:]).all() and np.isnan(lse[1:]).all()
    xd = _f64(x)
    ro, rl = O.decode(xd["q"][:1], xd["k"][:1], xd["v"][:1], [299], 1.0, 8)
    assert float(np.abs(out[:1] - ro).max()) <= TOL["bf16"]


def test_decode_equals_forward_row():
    """The decoding step at position i equals row i of fsa_forward on the same
    sequence (two different kernels)."""
    torch = _torch()
    from static_pattern_sparse_amd import fsa as F
    _say("decode vs forward")
    T = 1500
    seq = I.make_inputs(2, 2, T, 64, "bf16", 83, 0, with_dout=False)
    q, k, v = (I.to_device(seq[n], "bf16") for n in ("q", "k", "v"))
    alpha, W = float(np.float32(0.6333333)), 12
    out, lse = F.fsa_forward(q, k, v, alpha, W)
    for i in (0, 11, 12, 700, T - 1):
        pos = torch.full((2,), i, dtype=torch.int32, device="cuda")
        do, dl = F.fsa_decode(q[:, :, i].contiguous(), k, v, pos, alpha, W)
        torch.cuda.synchronize()
        assert float((do - out[:, :, i]).abs().max()) <= 2 * TOL["bf16"]
        assert float((dl - lse[:, :, i]).abs().max()) <= 2 * TOL["bf16"]


def test_workload_decode_t4096():
    """The decoding workload at full size, every layer's schedule value."""
    w = I.WORKLOADS["decode16_bf16_b8h8t4096d64_w12"]
    alphas = O.schedule(O.SCHEDULE_LINEAR, w.layers)
    for layer in (0, 1, 7, 15):
        _say(w.name, layer)
        x = I.decode_inputs(w, layer)
        check_decode(x, w.dtype, float(alphas[layer]), 12)


def test_decode_bf16_out():
    """FSA_OUT_BF16 in the decoding step: the fp32 result rounded to nearest
    even, bit for bit."""
    torch = _torch()
    from static_pattern_sparse_amd import fsa as F
    _say("decode bf16 out")
    x = I.make_decode_inputs(4, 2, 1200, 64, "bf16", 84, 0, [1199, 700, 12, 0])
    q, k, v = (I.to_device(x[n], "bf16") for n in ("q", "k", "v"))
    pos = torch.from_numpy(x["pos"]).to("cuda")
    o32, l32 = F.fsa_decode(q, k, v, pos, 0.8, 12)
    ob, lb = F.fsa_decode(q, k, v, pos, 0.8, 12, out_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    assert ob.dtype == torch.bfloat16
    assert torch.equal(ob, o32.to(torch.bfloat16)) and torch.equal(lb, l32)


def _draw_decode(seed):
    r = np.random.default_rng(90000 + seed)
    B, H = int(r.integers(1, 6)), int(r.integers(1, 4))
    T = int(r.integers(1, 3000))
    D = int(r.choice([64, 128]))
    dtype = "f32" if r.random() < 0.3 else "bf16"
    alpha = float(np.float32(r.uniform(0.5, 1.5)))
    W = int(r.integers(1, 80))
    pattern = str(r.choice(sorted(ORACLE_PATTERN)))
    pos = [int(p) for p in r.integers(0, T, B)]
    return B, H, T, D, dtype, alpha, W, pattern, pos


@pytest.mark.parametrize("seed", range(12))
def test_decode_random(seed):
    """Seeded random batch sizes, cache lengths, head dims, dtypes, windows,
    patterns and positions."""
    B, H, T, D, dtype, alpha, W, pattern, pos = _draw_decode(seed)
    _say("decode random", seed, B, H, T, D, dtype, alpha, W, pattern, pos)
    x = I.make_decode_inputs(B, H, T, D, dtype, 300 + seed % 7, 0, pos)
    check_decode(x, dtype, alpha, W, pattern)
