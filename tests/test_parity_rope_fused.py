"""GPU parity of RoPE fused into the attention kernels (fsa_forward_rope,
fsa_backward_rope) against the oracle's rotation followed by its attention:

  q_rot = bf16(oracle.rope(q_pre)), k_rot = bf16(oracle.rope(k_pre));
  out, lse = oracle.forward(q_rot, k_rot, v);
  dq, dk, dv, dalpha = oracle.backward(q_rot, k_rot, v, dout);
  dq_pre = oracle.rope(dq, inverse), dk_pre = oracle.rope(dk, inverse).

The kernels take q_pre and k_rot (the key rows keep their pass), turn the
query tile in registers, hand the turned rows on, and turn dq and dk back at
store time. Tolerances as test_parity; the turned query rows are the oracle's
rounded to bf16 exactly, or one bf16 step (of the larger value) apart where
the fp32 rotation lands next to a rounding midpoint (at most 1 in 1000
elements).
[Depth-Staggered Fibonacci Spacing for Sparse Attention: Methodology >
Architecture and attention > Implementation (RoPE before the gather)]
"""

from __future__ import annotations

import numpy as np
import pytest

from oracle import fsa_oracle as O
from static_pattern_sparse_amd import inputs as I
from tests.test_parity import DALPHA_RTOL, TOL, _say

pytestmark = pytest.mark.gpu


def _torch():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch


def _bf16(x):
    return I.round_to_bf16(np.asarray(x, dtype=np.float64).astype(np.float32))


CASES = [
    # B, H, T, D, alpha, W, base, pos0
    (1, 2, 700, 64, 0.8333333, 12, 10000.0, None),
    (2, 2, 333, 128, 1.2913, 6, 10000.0, (0, 1000)),
    (2, 1, 1031, 64, 0.5, 12, 500000.0, (60000, 4097)),      # far positions
    (1, 3, 45, 64, 1.5, 3, 10000.0, None),
]


@pytest.mark.parametrize("B,H,T,D,alpha,W,base,pos0", CASES)
def test_fused_rope_forward_backward(B, H, T, D, alpha, W, base, pos0):
    torch = _torch()
    from static_pattern_sparse_amd import fsa as F
    _say("fused rope", B, H, T, D, alpha, W, base, pos0)
    alpha = float(np.float32(alpha))
    wid = 500 + T
    pre = {n: I.make_tensor(B, H, T, D, "bf16", wid, 0, n, None)
           for n in ("q", "k", "v", "dout")}
    p0 = None if pos0 is None else np.array(pos0, dtype=np.int64)
    q_rot = _bf16(O.rope(pre["q"].astype(np.float64), base, p0))
    k_rot = _bf16(O.rope(pre["k"].astype(np.float64), base, p0))
    dev = lambda a: I.to_device(a, "bf16")
    pos_t = None if pos0 is None else torch.tensor(pos0, dtype=torch.int32, device="cuda")
    qg, kg, vg, gg = dev(pre["q"]), dev(k_rot), dev(pre["v"]), dev(pre["dout"])
    out = torch.full((B, H, T, D), float("nan"), device="cuda")
    lse = torch.full((B, H, T), float("nan"), device="cuda")
    out, lse, qr = F.fsa_forward_rope(qg, kg, vg, alpha, W, base, pos0=pos_t, out=out, lse=lse)
    nan = lambda: torch.full((B, H, T, D), float("nan"), device="cuda")
    dq, dk, dv = nan(), nan(), nan()
    da = torch.full((1,), float("nan"), device="cuda")
    F.fsa_backward_rope(qr, kg, vg, gg, lse, alpha, W, base, pos0=pos_t, dq=dq, dk=dk,
                        dv=dv, dalpha=da)
    torch.cuda.synchronize()
    # the turned query rows the forward hands on
    got_q = qr.float().cpu().numpy()
    diff = np.abs(got_q - q_rot)
    # one bf16 step of the larger value (a result next to a power of two may
    # round into the binade above), plus the fp32 rotation's absolute error,
    # a few fp32 steps of the operands (order 1): it dominates where the two
    # products cancel to a result near 0 (the bound of the RoPE pass's test)
    step = np.maximum(np.abs(q_rot), np.abs(got_q)) * 2.0 ** -7 + 2e-6
    assert float((diff > step).mean()) == 0.0, float(diff.max())
    assert float((diff > 0).mean()) <= 1e-3
    # attention on the turned rows, and the gradients turned back
    xd = lambda a: np.asarray(a, dtype=np.float64)
    ro, rl = O.forward(xd(q_rot), xd(k_rot), xd(pre["v"]), alpha, W)
    rq, rk, rv, ra = O.backward(xd(q_rot), xd(k_rot), xd(pre["v"]), xd(pre["dout"]), alpha, W)
    rq = O.rope(rq, base, p0, inverse=True)
    rk = O.rope(rk, base, p0, inverse=True)
    tol = TOL["bf16"]
    for name, g, r in (("out", out, ro), ("lse", lse, rl), ("dq_pre", dq, rq),
                       ("dk_pre", dk, rk), ("dv", dv, rv)):
        a = g.double().cpu().numpy()
        assert np.isfinite(a).all(), name
        e = float(np.abs(a - r).max())
        assert e <= tol, f"{name} err {e}"
    assert abs(float(da.item()) - ra) <= DALPHA_RTOL * abs(ra)


@pytest.mark.parametrize("D,pos", [(64, None), (128, (3, 70000))])
def test_fused_equals_separate_passes_bitwise(D, pos):
    """The fused calls turn by the same bits as the RoPE pass (the same angle
    formula, in the same order), so the fused forward and backward give
    exactly what the separate passes around the plain calls give: turned
    query rows, out, lse, the turned-back dq and dk, dv and dalpha."""
    torch = _torch()
    from static_pattern_sparse_amd import fsa as F
    _say("fused vs separate passes", D, pos)
    B, H, T, alpha, W, base = 2, 3, 900, 0.7317, 12, 10000.0
    pre = {n: I.make_tensor(B, H, T, D, "bf16", 611, 0, n, None)
           for n in ("q", "k", "v", "dout")}
    qg, kpre, vg, gg = (I.to_device(pre[n], "bf16") for n in ("q", "k", "v", "dout"))
    p0 = None if pos is None else torch.tensor(pos, dtype=torch.int32, device="cuda")
    kg = F.fsa_rope(kpre, base, pos0=p0)
    o1, l1, qr = F.fsa_forward_rope(qg, kg, vg, alpha, W, base, pos0=p0)
    g1 = F.fsa_backward_rope(qr, kg, vg, gg, l1, alpha, W, base, pos0=p0)
    qs = F.fsa_rope(qg, base, pos0=p0)
    o2, l2 = F.fsa_forward(qs, kg, vg, alpha, W)
    dq, dk, dv, da = F.fsa_backward(qs, kg, vg, gg, l2, alpha, W)
    dq = F.fsa_rope(dq, base, pos0=p0, inverse=True)
    dk = F.fsa_rope(dk, base, pos0=p0, inverse=True)
    torch.cuda.synchronize()
    assert torch.equal(qr, qs)
    assert torch.equal(o1, o2) and torch.equal(l1, l2)
    for name, a, b in zip(("dq_pre", "dk_pre", "dv", "dalpha"), g1, (dq, dk, dv, da)):
        assert torch.equal(a, b), name
