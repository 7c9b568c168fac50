"""GPU parity of the RoPE pass (fsa_rope, through the C ABI) against the fp64
oracle's rope (reading R12).

Bars:
* fp32 output: max |GPU - oracle| <= 1e-5 (the angle is reduced in fp64 and
  rotated in fp32: about 3e-7 relative to |x| <= 6 for N(0, 1) inputs).
* bf16 output: the GPU rounds its fp32 result to bf16, nearest even. The
  reference is the oracle's fp64 result rounded the same way (to fp32, then to
  bf16). The GPU's fp32 value carries the rotation's own error (at most about
  4e-7 absolute for these inputs), so a value that close to a bf16 rounding
  midpoint may round the other way: every element must agree within one bf16
  ulp plus 2e-6 absolute (the absolute part matters only for values near 0,
  where the two products of the rotation cancel), and at most 1e-3 of the
  elements may differ at all.
Outputs are filled with NaN before each launch, so an element the kernel
fails to write cannot pass.
"""

from __future__ import annotations

import sys

import numpy as np
import pytest

from oracle import fsa_oracle as O
from static_pattern_sparse_amd import inputs as I

pytestmark = pytest.mark.gpu

TOL_F32 = 1e-5
ABS_BF16 = 2e-6
MAX_FLIP_FRACTION = 1e-3


def _torch():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch


def _say(*a):
    print("[case]", *a, flush=True)
    sys.stdout.flush()


def _tdt(name):
    import torch
    return {"f32": torch.float32, "bf16": torch.bfloat16}[name]


def _bf16_of(x64):
    return I.round_to_bf16(np.asarray(x64, dtype=np.float64).astype(np.float32)).astype(np.float64)


def check_close(got, ref64, out_dtype):
    """got: GPU result as float64; ref64: the oracle's fp64 result."""
    assert np.isfinite(got).all()
    if out_dtype == "f32":
        err = float(np.abs(got - ref64).max())
        assert err <= TOL_F32, f"max err {err}"
        return
    ref = _bf16_of(ref64)
    diff = got != ref
    ulp = np.maximum(np.abs(ref), np.abs(got)) * 2.0 ** -7     # one bf16 ulp bound
    bad = np.abs(got - ref) > ulp + ABS_BF16
    assert not bad.any(), (f"{int(bad.sum())} elements beyond one bf16 ulp + {ABS_BF16}: "
                           f"got {got[bad][:4]}, ref {ref[bad][:4]}")
    frac = float(diff.mean())
    assert frac <= MAX_FLIP_FRACTION, f"{frac:.2e} of the elements differ"


def gpu_rope(x_host, in_dtype, out_dtype, base, pos0=None, inverse=False, in_place=False):
    torch = _torch()
    from static_pattern_sparse_amd import fsa as F
    x = I.to_device(x_host, in_dtype)
    p = None if pos0 is None else torch.tensor(np.asarray(pos0, dtype=np.int32), device="cuda")
    if in_place:
        y = F.fsa_rope(x, base, p, inverse, out=x)
        assert y.data_ptr() == x.data_ptr()
    else:
        out = torch.full(x.shape, float("nan"), dtype=_tdt(out_dtype), device="cuda")
        y = F.fsa_rope(x, base, p, inverse, out=out)
    torch.cuda.synchronize()
    return y.float().cpu().double().numpy()


def _input(shape, dtype, seed):
    x = np.random.default_rng(seed).standard_normal(shape).astype(np.float32)
    return I.round_to_bf16(x) if dtype == "bf16" else x


CASES = [
    # B, H, T, D, in, out, base, pos0, inverse
    (2, 3, 37, 64, "bf16", "bf16", 10000.0, None, False),
    (2, 3, 37, 64, "f32", "f32", 10000.0, None, False),
    (2, 2, 19, 128, "f32", "bf16", 500000.0, [0, 65519], False),
    (3, 1, 23, 128, "bf16", "f32", 500000.0, [65535, 7, 1000000], False),
    (2, 2, 40, 64, "f32", "f32", 10000.0, [4000, -3], True),
    (1, 4, 9, 8, "f32", "f32", 10000.0, None, False),
    (1, 2, 11, 24, "bf16", "bf16", 10000.0, [123], True),
    (2, 1, 5, 256, "f32", "bf16", 10000.0, None, False),
    (4, 2, 1, 64, "bf16", "bf16", 10000.0, [4095, 4034, 3973, 0], False),   # decoding rows
    (2, 9, 7, 16, "bf16", "bf16", 10000.0, [5, 100], False),   # heads past one group of 8
    (1, 17, 5, 8, "f32", "f32", 500000.0, None, True),
]


@pytest.mark.parametrize("B,H,T,D,din,dout,base,pos0,inverse", CASES)
def test_rope_small(B, H, T, D, din, dout, base, pos0, inverse):
    _say("rope", B, H, T, D, din, dout, base, pos0, inverse)
    x = _input((B, H, T, D), din, 900 + D + T)
    got = gpu_rope(x, din, dout, base, pos0, inverse)
    ref = O.rope(x.astype(np.float64), base, pos0, inverse)
    check_close(got, ref, dout)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_rope_in_place(dtype):
    _say("rope in place", dtype)
    x = _input((2, 2, 33, 64), dtype, 951)
    got = gpu_rope(x, dtype, dtype, 10000.0, [17, 2048], in_place=True)
    check_close(got, O.rope(x.astype(np.float64), 10000.0, [17, 2048]), dtype)


def test_rope_inverse_round_trip_f32():
    """fp32 rows turned forward and back on the GPU return within 2e-6."""
    torch = _torch()
    from static_pattern_sparse_amd import fsa as F
    _say("rope round trip")
    x = torch.from_numpy(_input((2, 4, 300, 128), "f32", 952)).cuda()
    pos = torch.tensor([0, 60000], dtype=torch.int32, device="cuda")
    y = F.fsa_rope(F.fsa_rope(x, 500000.0, pos), 500000.0, pos, inverse=True)
    torch.cuda.synchronize()
    assert float((y - x).abs().max()) <= 2e-6


def test_rope_workload_t1024_all_rows():
    """The pass over one layer's pre-RoPE q at the training size, B8 H8 T1024
    D64, bf16 to bf16, every element against the oracle."""
    _say("rope t1024")
    w = I.WORKLOADS["linear16_bwd_bf16_b8h8t1024d64_w12"]
    x = I.make_tensor(w.B, w.H, w.T, w.D, "bf16", w.workload_id, 0, "q", None)
    got = gpu_rope(x, "bf16", "bf16", w.rope_base)
    check_close(got, O.rope(x.astype(np.float64), w.rope_base), "bf16")


def test_rope_workload_t65536_sampled_rows():
    """The 65536-token size (B1 H16 D128, base 500000), bf16 to bf16: the
    launch covers every row; sampled rows, the last ones included, are checked
    against the oracle row by row."""
    torch = _torch()
    from static_pattern_sparse_amd import fsa as F
    _say("rope t65536")
    w = I.WORKLOADS["linear16_bf16_b1h16t65536d128_w12"]
    rng = np.random.default_rng(953)
    x = torch.from_numpy(I.round_to_bf16(
        rng.standard_normal((w.B, w.H, w.T, w.D)).astype(np.float32))).to(torch.bfloat16).cuda()
    y = F.fsa_rope(x, w.rope_base)
    torch.cuda.synchronize()
    rows = np.concatenate([[0, 1, 4095, 32768], rng.integers(0, w.T, 60), [w.T - 2, w.T - 1]])
    xs = x[:, :, rows].float().cpu().double().numpy()          # [1, H, R, D]
    ys = y[:, :, rows].float().cpu().double().numpy()
    for r, t in enumerate(rows):
        ref = O.rope(xs[:, :, r:r + 1], w.rope_base, [int(t)])
        check_close(ys[:, :, r:r + 1], ref, "bf16")


def test_rope_then_forward():
    """Pre-RoPE q and k through fsa_rope and fsa_forward match the oracle's
    rope followed by the oracle's forward (bf16 rows, tolerance 2e-3)."""
    torch = _torch()
    from static_pattern_sparse_amd import fsa as F
    _say("rope then forward")
    B, H, T, D, base, alpha, W = 2, 2, 400, 64, 10000.0, float(np.float32(0.7317)), 12
    q0, k0 = _input((B, H, T, D), "bf16", 954), _input((B, H, T, D), "bf16", 955)
    v = _input((B, H, T, D), "bf16", 956)
    qr = F.fsa_rope(I.to_device(q0, "bf16"), base)
    kr = F.fsa_rope(I.to_device(k0, "bf16"), base)
    out, lse = F.fsa_forward(qr, kr, I.to_device(v, "bf16"), alpha, W)
    torch.cuda.synchronize()
    rq = _bf16_of(O.rope(q0.astype(np.float64), base))
    rk = _bf16_of(O.rope(k0.astype(np.float64), base))
    ro, rl = O.forward(rq, rk, v.astype(np.float64), alpha, W)
    assert float(np.abs(out.cpu().double().numpy() - ro).max()) <= 2e-3
    assert float(np.abs(lse.cpu().double().numpy() - rl).max()) <= 2e-3


def test_rope_inverse_carries_gradients():
    """The gradient of a loss with respect to pre-RoPE q is the inverse pass
    applied to fsa_backward's dq (fp32 to fp32), against the oracle's inverse
    of the same dq."""
    torch = _torch()
    from static_pattern_sparse_amd import fsa as F
    _say("rope inverse of dq")
    B, H, T, D, base, alpha, W = 1, 2, 300, 64, 10000.0, 1.0, 8
    x = I.make_inputs(B, H, T, D, "bf16", 957, 0)
    q, k, v, do = (I.to_device(x[n], "bf16") for n in ("q", "k", "v", "dout"))
    _, lse = F.fsa_forward(q, k, v, alpha, W)
    dq, dk, dv, da = F.fsa_backward(q, k, v, do, lse, alpha, W)
    pos = torch.tensor([11], dtype=torch.int32, device="cuda")
    g = F.fsa_rope(dq, base, pos, inverse=True)
    torch.cuda.synchronize()
    ref = O.rope(dq.cpu().double().numpy(), base, [11], inverse=True)
    scale = max(1.0, float(np.abs(ref).max()))
    assert float(np.abs(g.cpu().double().numpy() - ref).max()) <= TOL_F32 * scale
