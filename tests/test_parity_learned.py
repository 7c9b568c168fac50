"""GPU parity of the learned-alpha path through the C ABI (reading R16):

* fsa_theta_alpha: alpha against the oracle's map (fp64, rounded once), and
  each layer's device tap table, bit for bit, against the table the oracle's
  offset table fixes for that alpha (kept terms ascending; fp32 weights
  1 - t and t rounded once from the exact distance; slope -f or 0);
* fsa_forward_dev / fsa_backward_dev read the device table and give exactly
  what fsa_forward_ex / fsa_backward_ex give for the same alpha on the host;
* fsa_theta_step: one update after another against the oracle's update from
  the same fp32 state (theta, m, v within one fp32 ulp, the count exact);
* a whole learned step (forward, backward of three layers, the update)
  against the oracle's forward, backward and update.
[Depth-Staggered Fibonacci Spacing for Sparse Attention: Methodology >
Experimental variables, Learned; Architecture and attention > Scaling]
"""

from __future__ import annotations

import numpy as np
import pytest

from oracle import fsa_oracle as O
from static_pattern_sparse_amd import inputs as I
from tests.test_parity import TOL, DALPHA_RTOL, _say

pytestmark = pytest.mark.gpu

MAPS = {"clamp": O.THETA_CLAMP, "tanh": O.THETA_TANH}
PATTERNS = {0: ("fib", "lerp"), 1: ("pow2", "lerp"), 2: ("fib", "round"), 3: ("pow2", "round")}


def _torch():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch


def _parse(rec):
    """A device tap record (struct of int n, int c[15], float w_lo[15],
    w_hi[15], neg_f[15]) as numpy arrays."""
    b = np.ascontiguousarray(rec[:244])
    n = int(b[:4].view(np.int32)[0])
    c = b[4:64].view(np.int32)
    w = b[64:244].view(np.float32).reshape(3, 15)
    return n, c, w[0], w[1], w[2]


def _expected(alpha, W, pattern):
    base, mode = PATTERNS[pattern]
    tab = O.offset_table(alpha, W, base=base, mode=mode)
    keep = np.nonzero(tab.keep)[0]
    c = np.zeros(15, np.int32)
    wl, wh, nf = (np.zeros(15, np.float32) for _ in range(3))
    for j, k in enumerate(keep):
        c[j] = tab.c[k]
        wh[j] = np.float32(tab.t[k])
        wl[j] = np.float32(1.0 - tab.t[k])
        nf[j] = np.float32(tab.slope[k])
    return len(keep), c, wl, wh, nf


@pytest.mark.parametrize("map_name", sorted(MAPS))
@pytest.mark.parametrize("W,pattern", [(12, 0), (1, 0), (6, 1), (12, 2), (30, 3)])
def test_theta_alpha_and_tables(map_name, W, pattern):
    torch = _torch()
    from static_pattern_sparse_amd import fsa as F
    _say("theta_alpha", map_name, W, pattern)
    mp = MAPS[map_name]
    r = np.random.default_rng(W + 10 * pattern)
    lo, hi = (0.2, 1.8) if mp == O.THETA_CLAMP else (-3.0, 3.0)
    th = np.concatenate([r.uniform(lo, hi, 60), [O.theta_init(mp), 0.5, 1.5, -0.0]])
    th = th.astype(np.float32)
    theta = torch.from_numpy(th).cuda()
    alpha, tables = F.fsa_theta_alpha(theta, mp, W, pattern)
    torch.cuda.synchronize()
    a = alpha.cpu().numpy()
    recs = tables.cpu().numpy()
    for l in range(len(th)):
        ref = O.alpha_of_theta(float(th[l]), mp)
        if mp == O.THETA_CLAMP:
            assert a[l] == ref
        else:                                   # the fp64 tanh may differ by an ulp
            assert abs(a[l] - ref) <= np.spacing(np.float32(ref)), (th[l], a[l], ref)
        got, exp = _parse(recs[l]), _expected(float(a[l]), W, pattern)
        assert got[0] == exp[0], (l, got[0], exp[0])
        for g, e in zip(got[1:], exp[1:]):
            assert np.array_equal(g.view(np.uint32), e.view(np.uint32)), (l, g, e)
    assert float(alpha[len(th) - 4].item()) == 1.0        # theta_init gives alpha 1


@pytest.mark.parametrize("D,dtype", [(64, "bf16"), (128, "bf16"), (64, "f32")])
def test_device_table_equals_host_alpha(D, dtype):
    torch = _torch()
    from static_pattern_sparse_amd import fsa as F
    _say("device table vs host alpha", D, dtype)
    B, H, T, W = 1, 3, 700, 10
    theta = torch.tensor([0.3, -0.8], dtype=torch.float32, device="cuda")
    alpha, tables = F.fsa_theta_alpha(theta, F.FSA_THETA_TANH, W)
    x = I.make_inputs(B, H, T, D, dtype, 410, 0)
    q, k, v, g = (I.to_device(x[n], dtype) for n in ("q", "k", "v", "dout"))
    for l in range(2):
        a = float(alpha[l].item())
        o1, l1 = F.fsa_forward(q, k, v, a, W)
        o2, l2 = F.fsa_forward_dev(q, k, v, tables[l], W)
        g1 = F.fsa_backward(q, k, v, g, l1, a, W)
        g2 = F.fsa_backward_dev(q, k, v, g, l2, tables[l], W)
        torch.cuda.synchronize()
        assert torch.equal(o1, o2) and torch.equal(l1, l2)
        for t1, t2 in zip(g1, g2):
            assert torch.equal(t1, t2)


def _state(torch, L, step=0):
    st = torch.zeros(8 * L + 16, dtype=torch.uint8, device="cuda")
    return st


def _unpack(state, L):
    b = state.cpu().numpy()
    f = b[:8 * L].view(np.float32)
    return f[:L].copy(), f[L:2 * L].copy(), int(b[8 * L:8 * L + 4].view(np.int32)[0])


def _ulp_close(got, ref):
    ref32 = np.float32(ref)
    return abs(np.float64(got) - ref) <= np.spacing(np.abs(ref32)) + 1e-30


@pytest.mark.parametrize("map_name", sorted(MAPS))
@pytest.mark.parametrize("opt", ["sgd", "adam"])
def test_theta_step_vs_oracle(map_name, opt):
    torch = _torch()
    from static_pattern_sparse_amd import fsa as F
    _say("theta_step", map_name, opt)
    mp = MAPS[map_name]
    op = {"sgd": O.OPT_SGD, "adam": O.OPT_ADAM}[opt]
    L, W = 16, 12
    r = np.random.default_rng(7 + op + 2 * mp)
    lo, hi = (0.45, 1.55) if mp == O.THETA_CLAMP else (-2.0, 2.0)
    th = r.uniform(lo, hi, L).astype(np.float32)
    theta = torch.from_numpy(th).cuda()
    state = _state(torch, L)
    alpha = torch.empty(L, dtype=torch.float32, device="cuda")
    tables = torch.empty((L, 256), dtype=torch.uint8, device="cuda")
    lr = float(np.float32(0.05 if op == O.OPT_SGD else 0.01))
    b1, b2, eps = (float(np.float32(x)) for x in (0.9, 0.999, 1e-8))
    m = np.zeros(L, np.float32)
    v = np.zeros(L, np.float32)
    for s in range(5):
        da = (r.standard_normal(L) * 3).astype(np.float32)
        prev = theta.cpu().numpy()
        F.fsa_theta_step(theta, torch.from_numpy(da).cuda(), mp, op, lr, state, alpha, tables,
                         W, beta1=b1, beta2=b2, eps=eps)
        torch.cuda.synchronize()
        ref_th, ref_m, ref_v, _ = O.theta_step(prev, da, m, v, s, mp, op, lr, b1, b2, eps)
        got_th = theta.cpu().numpy()
        gm, gv, count = _unpack(state, L)
        assert count == s + 1
        for l in range(L):
            assert _ulp_close(got_th[l], ref_th[l]), (s, l, got_th[l], ref_th[l])
            if op == O.OPT_ADAM:
                assert _ulp_close(gm[l], ref_m[l]) and _ulp_close(gv[l], ref_v[l])
        a = alpha.cpu().numpy()
        for l in range(L):
            ref = O.alpha_of_theta(float(got_th[l]), mp)
            assert abs(a[l] - ref) <= (0 if mp == O.THETA_CLAMP else np.spacing(np.float32(ref)))
        m, v = gm, gv


@pytest.mark.parametrize("map_name", sorted(MAPS))
def test_learned_step_vs_oracle(map_name):
    """theta -> alpha -> forward and backward of three layers (device tables)
    -> one gradient-descent update, against the oracle's forward, backward
    (at the GPU's fp32 alpha) and update."""
    torch = _torch()
    from static_pattern_sparse_amd import fsa as F
    _say("learned step", map_name)
    mp = MAPS[map_name]
    L, B, H, T, D, W = 3, 1, 2, 600, 64, 8
    th0 = np.array([O.theta_init(mp), O.theta_init(mp) + 0.21, O.theta_init(mp) - 0.33],
                   dtype=np.float32)
    theta = torch.from_numpy(th0).cuda()
    alpha, tables = F.fsa_theta_alpha(theta, mp, W)
    dalpha = torch.full((L,), float("nan"), device="cuda")
    xs = [I.make_inputs(B, H, T, D, "bf16", 420, l) for l in range(L)]
    ref_da = []
    for l in range(L):
        x = xs[l]
        q, k, v, g = (I.to_device(x[n], "bf16") for n in ("q", "k", "v", "dout"))
        out, lse = F.fsa_forward_dev(q, k, v, tables[l], W)
        F.fsa_backward_dev(q, k, v, g, lse, tables[l], W, dalpha=dalpha[l:l + 1])
        a = float(alpha[l].item())
        xd = {n: t.astype(np.float64) for n, t in x.items()}
        ro, _ = O.forward(xd["q"], xd["k"], xd["v"], a, W)
        assert float(np.abs(out.cpu().double().numpy() - ro).max()) <= TOL["bf16"]
        ref_da.append(O.backward(xd["q"], xd["k"], xd["v"], xd["dout"], a, W)[3])
    torch.cuda.synchronize()
    got_da = dalpha.cpu().numpy()
    for l in range(L):
        assert abs(got_da[l] - ref_da[l]) <= DALPHA_RTOL * abs(ref_da[l])
    lr = float(np.float32(0.002))
    state = _state(torch, L)
    F.fsa_theta_step(theta, dalpha, mp, F.FSA_OPT_SGD, lr, state, alpha, tables, W)
    torch.cuda.synchronize()
    ref_th, _, _, ref_g = O.theta_step(th0, ref_da, [0] * L, [0] * L, 0, mp, O.OPT_SGD, lr)
    got = theta.cpu().numpy()
    for l in range(L):
        assert abs(got[l] - ref_th[l]) <= lr * abs(ref_g[l]) * 2e-3 + np.spacing(np.float32(1.5))
    assert not np.array_equal(got, th0)           # the update moved theta
