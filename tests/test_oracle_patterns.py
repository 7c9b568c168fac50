"""Pins of the oracle's other tap patterns: the power-of-two base and the
rounded (mask) mode.

Source page: Depth-Staggered Fibonacci Spacing for Sparse Attention
(gist.science technical summary): Methodology > Control variables (the
power-of-two control base), Core contributions and results > 2. Learned
dilation is inert (static runs take integer offsets through a fused mask) and
> 3. Length extrapolation (offsets 1024 and 2048 first met at 4096 tokens).
Every test runs on the CPU; the references are independent dense forms
(`tests/dense_forms.py`) and exact rational arithmetic.
"""

from __future__ import annotations

import math
from fractions import Fraction

import numpy as np
import pytest
import torch

from oracle import fsa_oracle as O
from tests import dense_forms as DF

BASE_LISTS = {"fib": DF.FIB_LIST, "pow2": DF.POW2_LIST}


def _rand(shape, seed):
    return np.random.default_rng(seed).standard_normal(shape)


def _nearest_even(x: Fraction) -> int:
    """Nearest integer to a non-negative rational, ties to the even one."""
    fl = x.numerator // x.denominator
    r = x - fl
    if r > Fraction(1, 2):
        return fl + 1
    if r < Fraction(1, 2):
        return fl
    return fl if fl % 2 == 0 else fl + 1


def _rounded_distances(alpha, W, base):
    a = Fraction(float(np.float32(alpha)))
    return [_nearest_even(a * f) for f in BASE_LISTS[base] if a * f >= W]


# ---------------------------------------------------------------- tables
def test_pow2_base_terms():
    # fifteen powers of two; 1024 and 2048 (the page's late offsets) included
    assert O.POW2 == tuple(DF.POW2_LIST)
    assert len(O.POW2) == len(O.FIB) == 15
    assert 1024 in O.POW2 and 2048 in O.POW2


@pytest.mark.parametrize("base", ["fib", "pow2"])
@pytest.mark.parametrize("alpha", [1.0, 0.5, 1.5, 0.7317, 1.2913, 0.5666667])
def test_tables_exact(base, alpha):
    a = Fraction(float(np.float32(alpha)))
    lerp = O.offset_table(alpha, 12, base=base, mode="lerp")
    rnd = O.offset_table(alpha, 12, base=base, mode="round")
    for n, f in enumerate(BASE_LISTS[base]):
        d = a * f
        assert Fraction(float(lerp.d[n])) == d
        assert Fraction(int(lerp.c[n])) - Fraction(float(lerp.t[n])) == d
        assert 0.0 <= lerp.t[n] < 1.0 and lerp.slope[n] == -f
        assert int(rnd.c[n]) == _nearest_even(d)
        assert abs(Fraction(int(rnd.c[n])) - d) <= Fraction(1, 2)
        assert rnd.t[n] == 0.0 and rnd.slope[n] == 0.0
        assert lerp.keep[n] == rnd.keep[n] == (d >= 12)


def test_round_ties_go_to_even():
    # alpha = 0.5: every odd Fibonacci term lands on a half; worked by hand
    # 0.5*(1,2,3,5,8,13,21,34,55,89,144,233,377,610,987)
    #   = 0.5 1 1.5 2.5 4 6.5 10.5 17 27.5 44.5 72 116.5 188.5 305 493.5
    expect = [0, 1, 2, 2, 4, 6, 10, 17, 28, 44, 72, 116, 188, 305, 494]
    assert list(O.offset_table(0.5, 12, mode="round").c) == expect


def test_unknown_pattern_rejected():
    with pytest.raises(ValueError):
        O.offset_table(1.0, 12, base="pow3")
    with pytest.raises(ValueError):
        O.offset_table(1.0, 12, mode="nearest")


# ---------------------------------------------------------------- rounded mode
def _dense_ref(q, k, v, g, dists, W):
    T = q.shape[0]
    tq, tk, tv = (torch.from_numpy(x).requires_grad_(True) for x in (q, k, v))
    out, lse = DF.dense_masked(tq, tk, tv, DF.attended_sets(T, W, dists))
    (out * torch.from_numpy(g)).sum().backward()
    return (out.detach().numpy(), lse.detach().numpy(), tq.grad.numpy(),
            tk.grad.numpy(), tv.grad.numpy())


@pytest.mark.parametrize("base", ["fib", "pow2"])
@pytest.mark.parametrize("alpha,W,T", [(0.7317, 4, 300), (1.2913, 6, 400),
                                       (0.5, 6, 350), (1.5, 12, 300),
                                       (0.5666667, 12, 520)])
def test_round_mode_equals_dense_masked(base, alpha, W, T):
    """Rounded offsets are a plain mask: forward and (dq, dk, dv) equal dense
    masked attention over {i-W+1..i} and {i - round(alpha*f)}; dalpha is 0."""
    D = 8
    dists = _rounded_distances(alpha, W, base)
    assert len(set(dists)) == len(dists)     # no two terms share a row here
    q, k, v, g = (_rand((T, D), s) for s in (200, 201, 202, 203))
    a = float(np.float32(alpha))
    out, lse = O.forward_slab(q, k, v, a, W, base=base, mode="round")
    dq, dk, dv, da, _ = O.backward_slab(q, k, v, g, a, W, base=base, mode="round")
    ro, rl, rq, rk, rv = _dense_ref(q, k, v, g, dists, W)
    np.testing.assert_allclose(out, ro, atol=1e-12, rtol=0)
    np.testing.assert_allclose(lse, rl, atol=1e-12, rtol=0)
    np.testing.assert_allclose(dq, rq, atol=1e-11, rtol=0)
    np.testing.assert_allclose(dk, rk, atol=1e-11, rtol=0)
    np.testing.assert_allclose(dv, rv, atol=1e-11, rtol=0)
    assert da == 0.0


def test_round_mode_loss_flat_in_alpha():
    """The attended rows of the rounded mode do not move for a small change of
    alpha (away from a rounding boundary), so the loss is unchanged: dalpha = 0
    is the true derivative there."""
    T, D, W, alpha = 300, 8, 4, 0.7317
    q, k, v, g = (_rand((T, D), s) for s in (210, 211, 212, 213))
    h = 1e-6
    for f in O.FIB:
        frac = (alpha * f) % 1.0
        assert abs(frac - 0.5) > 20 * h * f
    loss = []
    for a in (alpha - h, alpha, alpha + h):
        tab = O.offset_table(a, W, round_alpha_to_fp32=False, mode="round")
        out, _ = O.forward_slab(q, k, v, a, W, table=tab)
        loss.append(float((out * g).sum()))
    assert loss[0] == loss[1] == loss[2]


def test_round_equals_lerp_at_integer_distances():
    """At alpha = 1 every distance is an integer: the two modes attend the same
    rows with the same weights, bit for bit, and differ only in dalpha."""
    T, D, W = 400, 8, 6
    q, k, v, g = (_rand((T, D), s) for s in (220, 221, 222, 223))
    for base in ("fib", "pow2"):
        lo, ll = O.forward_slab(q, k, v, 1.0, W, base=base, mode="lerp")
        ro, rl = O.forward_slab(q, k, v, 1.0, W, base=base, mode="round")
        assert np.array_equal(lo, ro) and np.array_equal(ll, rl)
        gl = O.backward_slab(q, k, v, g, 1.0, W, base=base, mode="lerp")
        gr = O.backward_slab(q, k, v, g, 1.0, W, base=base, mode="round")
        for x, y in zip(gl[:3], gr[:3]):
            assert np.array_equal(x, y)
        assert gr[3] == 0.0 and gl[3] != 0.0


# ---------------------------------------------------------------- power-of-two base
@pytest.mark.parametrize("T,W", [(300, 8), (1100, 12), (70, 3)])
def test_pow2_alpha1_equals_dense_bruteforce(T, W):
    D = 8
    q, k, v, g = (_rand((T, D), s) for s in (230, 231, 232, 233))
    out, lse = O.forward_slab(q, k, v, 1.0, W, base="pow2")
    dq, dk, dv, _, _ = O.backward_slab(q, k, v, g, 1.0, W, base="pow2")
    ro, rl, rq, rk, rv = _dense_ref(q, k, v, g, DF.POW2_LIST, W)
    np.testing.assert_allclose(out, ro, atol=1e-12, rtol=0)
    np.testing.assert_allclose(lse, rl, atol=1e-12, rtol=0)
    np.testing.assert_allclose(dq, rq, atol=1e-11, rtol=0)
    np.testing.assert_allclose(dk, rk, atol=1e-11, rtol=0)
    np.testing.assert_allclose(dv, rv, atol=1e-11, rtol=0)


@pytest.mark.parametrize("alpha,W,T", [(0.7317, 4, 300), (1.2913, 6, 600),
                                       (0.5, 6, 300), (1.5, 3, 200)])
def test_pow2_lerp_equals_autograd_matrix_form(alpha, W, T):
    """Fractional power-of-two distances against the interpolation-matrix
    form, forward and every gradient including dalpha (autograd)."""
    D = 8
    q, k, v, g = (_rand((T, D), s) for s in (240, 241, 242, 243))
    a = float(np.float32(alpha))
    out, lse = O.forward_slab(q, k, v, a, W, base="pow2")
    dq, dk, dv, da, _ = O.backward_slab(q, k, v, g, a, W, base="pow2")
    tq, tk, tv = (torch.from_numpy(x).requires_grad_(True) for x in (q, k, v))
    ta = torch.tensor(a, dtype=torch.float64, requires_grad=True)
    ro, rl = DF.matrix_form(tq, tk, tv, ta, W, base_list=DF.POW2_LIST)
    (ro * torch.from_numpy(g)).sum().backward()
    np.testing.assert_allclose(out, ro.detach().numpy(), atol=1e-12, rtol=0)
    np.testing.assert_allclose(lse, rl.detach().numpy(), atol=1e-12, rtol=0)
    np.testing.assert_allclose(dq, tq.grad.numpy(), atol=1e-11, rtol=0)
    np.testing.assert_allclose(dk, tk.grad.numpy(), atol=1e-11, rtol=0)
    np.testing.assert_allclose(dv, tv.grad.numpy(), atol=1e-11, rtol=0)
    assert abs(da - float(ta.grad)) <= 1e-9 * max(1.0, abs(float(ta.grad)))


def test_pow2_dalpha_central_difference():
    T, D, W, alpha = 300, 8, 4, 0.7317
    q, k, v, g = (_rand((T, D), s) for s in (250, 251, 252, 253))
    h = 1e-7
    for f in O.POW2:
        frac = (alpha * f) % 1.0
        assert min(frac, 1 - frac) > 20 * h * f

    def loss(a):
        tab = O.offset_table(a, W, round_alpha_to_fp32=False, base="pow2")
        out, _ = O.forward_slab(q, k, v, a, W, table=tab)
        return float((out * g).sum())

    tab = O.offset_table(alpha, W, round_alpha_to_fp32=False, base="pow2")
    _, _, _, da, _ = O.backward_slab(q, k, v, g, alpha, W, table=tab)
    fd = (loss(alpha + h) - loss(alpha - h)) / (2 * h)
    assert abs(da - fd) <= 1e-5 * max(1.0, abs(fd))


@pytest.mark.parametrize("alpha,W", [(1.0, 8), (0.7317, 5), (1.5, 12)])
def test_pow2_q_zero_counts(alpha, W):
    """Q = 0: lse_i = ln n_i, with n_i = min(W, i+1) plus the kept terms whose
    lower row i - ceil(alpha*f) exists, counted in exact rationals."""
    T = 1100
    q = np.zeros((T, 4))
    k, v = _rand((T, 4), 260), _rand((T, 4), 261)
    _, lse = O.forward_slab(q, k, v, alpha, W, base="pow2")
    a = Fraction(float(np.float32(alpha)))
    ceil = [-((-a * f).numerator // (-a * f).denominator) for f in DF.POW2_LIST]
    kept = [c for c, f in zip(ceil, DF.POW2_LIST) if a * f >= W]
    n = np.array([min(W, i + 1) + sum(1 for c in kept if c <= i) for i in range(T)])
    np.testing.assert_allclose(lse, np.log(n), atol=1e-12, rtol=0)
    assert math.isclose(lse[1023], math.log(min(W, 1024) + len([c for c in kept if c <= 1023])))


def test_row_helpers_match_slabs_other_patterns():
    T, D, W, alpha = 600, 8, 5, 0.6333
    q, k, v, g = (_rand((T, D), s) for s in (270, 271, 272, 273))
    rows = np.array([0, 1, 4, 5, 6, 40, 211, 212, 599])
    for base, mode in (("pow2", "lerp"), ("fib", "round"), ("pow2", "round")):
        out, lse = O.forward_slab(q, k, v, alpha, W, base=base, mode=mode)
        dq, dk, dv, _, _ = O.backward_slab(q, k, v, g, alpha, W, base=base, mode=mode)
        ro, rl = O.forward_rows(q, k, v, alpha, W, rows, base=base, mode=mode)
        np.testing.assert_allclose(ro, out[rows], atol=1e-12, rtol=0)
        np.testing.assert_allclose(rl, lse[rows], atol=1e-12, rtol=0)
        rq, _ = O.dq_rows(q, k, v, g, alpha, W, rows, base=base, mode=mode)
        np.testing.assert_allclose(rq, dq[rows], atol=1e-12, rtol=0)
        rk, rv = O.dkdv_rows(q, k, v, g, alpha, W, rows, base=base, mode=mode)
        np.testing.assert_allclose(rk, dk[rows], atol=1e-12, rtol=0)
        np.testing.assert_allclose(rv, dv[rows], atol=1e-12, rtol=0)


# ---------------------------------------------------------------- planted mistakes
def test_pins_catch_floor_rounding(monkeypatch):
    """A rounded mode that truncated instead of rounding must fail the dense
    pin (planted in the oracle's table on the CPU)."""
    T, D, W, alpha = 300, 8, 4, 0.7317
    q, k, v, g = (_rand((T, D), s) for s in (280, 281, 282, 283))
    a = float(np.float32(alpha))
    tab = O.offset_table(a, W, mode="round")
    bad = tab._replace(c=np.floor(tab.d).astype(np.int64))
    assert not np.array_equal(bad.c, tab.c)
    out, _ = O.forward_slab(q, k, v, a, W, table=bad)
    ro, _, _, _, _ = _dense_ref(q, k, v, g, _rounded_distances(alpha, W, "fib"), W)
    assert float(np.abs(out - ro).max()) > 1e-3
