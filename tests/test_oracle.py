"""Pins of the fp64 oracle against what the page and the mathematics fix.

Every test here runs on the CPU. Source page: Depth-Staggered Fibonacci Spacing
for Sparse Attention (gist.science technical summary), sections Methodology >
Architecture and attention (attended set, scaling, interpolation, RoPE before
the gather) and Methodology > Experimental variables (schedules).
"""

from __future__ import annotations

import math
import os
from fractions import Fraction

import numpy as np
import pytest
import torch

from oracle import fsa_oracle as O
from tests import dense_forms as DF

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _rand(shape, seed):
    return np.random.default_rng(seed).standard_normal(shape)


def _load_rows(name):
    rows = []
    with open(os.path.join(GOLDEN, name)) as fh:
        for line in fh:
            line = line.strip()
            if line and not line.startswith("#"):
                rows.append(line.split())
    return rows


# ---------------------------------------------------------------- schedules
def test_schedule_fixed():
    a = O.schedule(O.SCHEDULE_FIXED, 16)
    assert a.dtype == np.float32 and (a == 1.0).all()


def test_schedule_linear_is_rounded_rational():
    a = O.schedule(O.SCHEDULE_LINEAR, 16)
    assert a[0] == np.float32(0.5) and a[15] == np.float32(1.5)
    assert (np.diff(a.astype(np.float64)) > 0).all()
    for l in range(16):
        exact = Fraction(1, 2) + Fraction(l, 15)
        # a[l] must be the float32 nearest to the exact rational
        v = Fraction(float(a[l]))
        up = Fraction(float(np.nextafter(a[l], np.float32(2))))
        dn = Fraction(float(np.nextafter(a[l], np.float32(0))))
        assert abs(v - exact) <= abs(up - exact)
        assert abs(v - exact) <= abs(dn - exact)


def test_schedule_coprime_golden_permutation():
    lin = O.schedule(O.SCHEDULE_LINEAR, 16)
    cop = O.schedule(O.SCHEDULE_COPRIME, 16)
    rows = _load_rows("coprime_perm_L16.txt")
    assert len(rows) == 16
    for layer, src in rows:
        assert cop[int(layer)] == lin[int(src)]
    assert sorted(cop.tolist()) == sorted(lin.tolist())
    # adjacent layers differ by 7 or 9 steps of the linear ladder
    pos = [int(s) for _, s in rows]
    gaps = {abs(pos[l + 1] - pos[l]) for l in range(15)}
    assert gaps <= {7, 9}


def test_schedule_rejects_bad_args():
    with pytest.raises(ValueError):
        O.schedule(O.SCHEDULE_COPRIME, 16, stride=4)
    with pytest.raises(ValueError):
        O.schedule(O.SCHEDULE_LINEAR, 0)


# ---------------------------------------------------------------- offsets
@pytest.mark.parametrize("alpha", [1.0, 0.5, 1.5, 0.7317, 1.2913])
def test_offset_table_exact(alpha):
    d, c, t, keep, slope = O.offset_table(alpha, 12)
    a = Fraction(float(np.float32(alpha)))
    for n, f in enumerate(O.FIB):
        assert Fraction(float(d[n])) == a * f          # exact product
        assert Fraction(int(c[n])) - Fraction(float(t[n])) == a * f
        assert 0.0 <= t[n] < 1.0
        assert keep[n] == (a * f >= 12)
        assert slope[n] == -f                          # position i - alpha*f


def test_offset_table_stagger_near_integer():
    # fp32(0.5 + 5/15) * 144 sits just below 120: the distance is fractional,
    # the lower row is i - 120 and the upper row i - 119 gets a tiny weight
    a = O.schedule(O.SCHEDULE_LINEAR, 16)[5]
    d, c, t, keep, _ = O.offset_table(a, 12)
    n = O.FIB.index(144)
    assert c[n] == 120 and 0.0 < t[n] < 1e-5


# ---------------------------------------------------------------- counts
def test_entry_counts_golden_q_zero():
    """Q = 0 makes every score 0, so lse_i = ln n_i and out_i = mean of the
    attended values; n_i is taken from the hand-derived fixture."""
    for alpha, W, i, n in _load_rows("entry_counts.txt"):
        alpha, W, i, n = float(alpha), int(W), int(i), int(n)
        T = max(i + 1, 16)
        q = np.zeros((T, 8))
        k = _rand((T, 8), 1)
        v = _rand((T, 8), 2)
        out, lse = O.forward_slab(q, k, v, alpha, W)
        assert abs(lse[i] - math.log(n)) < 1e-12


def test_q_zero_counts_match_set_enumeration():
    T, W = 1000, 8
    sets = DF.attended_sets(T, W, DF.FIB_LIST)
    q = np.zeros((T, 4))
    k = _rand((T, 4), 3)
    v = _rand((T, 4), 4)
    out, lse = O.forward_slab(q, k, v, 1.0, W)
    n = np.array([len(s) for s in sets])
    np.testing.assert_allclose(lse, np.log(n), atol=1e-12, rtol=0)
    mean = np.array([v[sorted(s)].mean(axis=0) for s in sets])
    np.testing.assert_allclose(out, mean, atol=1e-12, rtol=0)


# ---------------------------------------------------------------- forward pins
@pytest.mark.parametrize("T,W,D", [(300, 8, 16), (1100, 12, 8), (64, 3, 8)])
def test_alpha1_equals_dense_bruteforce(T, W, D):
    q, k, v = _rand((T, D), 10), _rand((T, D), 11), _rand((T, D), 12)
    out, lse = O.forward_slab(q, k, v, 1.0, W)
    sets = DF.attended_sets(T, W, DF.FIB_LIST)
    tq, tk, tv = (torch.from_numpy(x) for x in (q, k, v))
    ref_out, ref_lse = DF.dense_masked(tq, tk, tv, sets)
    np.testing.assert_allclose(out, ref_out.numpy(), atol=1e-12, rtol=0)
    np.testing.assert_allclose(lse, ref_lse.numpy(), atol=1e-12, rtol=0)


def test_window_covering_sequence_is_causal_attention():
    T, D = 200, 16
    q, k, v = _rand((T, D), 20), _rand((T, D), 21), _rand((T, D), 22)
    for alpha in (1.0, 0.7317):
        out, _ = O.forward_slab(q, k, v, alpha, T)
        ref = torch.nn.functional.scaled_dot_product_attention(
            torch.from_numpy(q)[None, None], torch.from_numpy(k)[None, None],
            torch.from_numpy(v)[None, None], is_causal=True)[0, 0]
        np.testing.assert_allclose(out, ref.numpy(), atol=1e-12, rtol=0)


@pytest.mark.parametrize("alpha,W,T", [(0.7317, 4, 200), (1.2913, 6, 400),
                                       (0.5, 6, 300), (1.5, 12, 300)])
def test_fractional_alpha_equals_matrix_form(alpha, W, T):
    D = 8
    q, k, v = _rand((T, D), 30), _rand((T, D), 31), _rand((T, D), 32)
    out, lse = O.forward_slab(q, k, v, alpha, W)
    a = torch.tensor(float(np.float32(alpha)), dtype=torch.float64)
    ref_out, ref_lse = DF.matrix_form(torch.from_numpy(q), torch.from_numpy(k),
                                      torch.from_numpy(v), a, W)
    np.testing.assert_allclose(out, ref_out.numpy(), atol=1e-12, rtol=0)
    np.testing.assert_allclose(lse, ref_lse.numpy(), atol=1e-12, rtol=0)


def test_stagger_values_equal_matrix_form():
    T, D = 260, 8
    q, k, v = _rand((T, D), 40), _rand((T, D), 41), _rand((T, D), 42)
    for alpha in O.schedule(O.SCHEDULE_LINEAR, 16)[::3]:
        out, lse = O.forward_slab(q, k, v, float(alpha), 12)
        a = torch.tensor(float(alpha), dtype=torch.float64)
        ref_out, _ = DF.matrix_form(torch.from_numpy(q), torch.from_numpy(k),
                                    torch.from_numpy(v), a, 12)
        np.testing.assert_allclose(out, ref_out.numpy(), atol=1e-12, rtol=0)


def test_normalisation_and_linearity():
    T, D, W, alpha = 500, 8, 6, 0.8123
    q, k = _rand((T, D), 50), _rand((T, D), 51)
    v1, v2 = _rand((T, D), 52), _rand((T, D), 53)
    ones = np.ones((T, D))
    out, _ = O.forward_slab(q, k, ones, alpha, W)
    np.testing.assert_allclose(out, 1.0, atol=1e-13, rtol=0)     # sum p = 1
    row = _rand((1, D), 54)
    out, _ = O.forward_slab(q, k, np.repeat(row, T, 0), alpha, W)
    np.testing.assert_allclose(out, np.repeat(row, T, 0), atol=1e-12, rtol=0)
    o1, _ = O.forward_slab(q, k, v1, alpha, W)
    o2, _ = O.forward_slab(q, k, v2, alpha, W)
    o12, _ = O.forward_slab(q, k, v1 + 2 * v2, alpha, W)
    np.testing.assert_allclose(o12, o1 + 2 * o2, atol=1e-12, rtol=0)


def test_batched_forward_matches_slabs():
    B, H, T, D = 2, 3, 64, 8
    q, k, v = _rand((B, H, T, D), 60), _rand((B, H, T, D), 61), _rand((B, H, T, D), 62)
    out, lse = O.forward(q, k, v, 0.9, 5)
    o, l = O.forward_slab(q[1, 2], k[1, 2], v[1, 2], 0.9, 5)
    assert np.array_equal(out[1, 2], o) and np.array_equal(lse[1, 2], l)


# ---------------------------------------------------------------- backward pins
def _autograd_matrix_form(q, k, v, dout, alpha, W):
    tq, tk, tv = (torch.from_numpy(x).requires_grad_(True) for x in (q, k, v))
    a = torch.tensor(float(alpha), dtype=torch.float64, requires_grad=True)
    out, _ = DF.matrix_form(tq, tk, tv, a, W)
    (out * torch.from_numpy(dout)).sum().backward()
    return tq.grad.numpy(), tk.grad.numpy(), tv.grad.numpy(), float(a.grad)


@pytest.mark.parametrize("alpha,W,T", [(1.0, 8, 300), (0.7317, 4, 200),
                                       (1.2913, 6, 300), (0.5, 6, 250)])
def test_backward_equals_autograd_matrix_form(alpha, W, T):
    D = 8
    q, k, v, g = (_rand((T, D), s) for s in (70, 71, 72, 73))
    alpha = float(np.float32(alpha))
    dq, dk, dv, da, _ = O.backward_slab(q, k, v, g, alpha, W)
    rq, rk, rv, ra = _autograd_matrix_form(q, k, v, g, alpha, W)
    np.testing.assert_allclose(dq, rq, atol=1e-11, rtol=0)
    np.testing.assert_allclose(dk, rk, atol=1e-11, rtol=0)
    np.testing.assert_allclose(dv, rv, atol=1e-11, rtol=0)
    assert abs(da - ra) <= 1e-9 * max(1.0, abs(ra))


def test_backward_alpha1_equals_dense_autograd():
    T, D, W = 400, 8, 8
    q, k, v, g = (_rand((T, D), s) for s in (80, 81, 82, 83))
    dq, dk, dv, _, _ = O.backward_slab(q, k, v, g, 1.0, W)
    tq, tk, tv = (torch.from_numpy(x).requires_grad_(True) for x in (q, k, v))
    out, _ = DF.dense_masked(tq, tk, tv, DF.attended_sets(T, W, DF.FIB_LIST))
    (out * torch.from_numpy(g)).sum().backward()
    np.testing.assert_allclose(dq, tq.grad.numpy(), atol=1e-11, rtol=0)
    np.testing.assert_allclose(dk, tk.grad.numpy(), atol=1e-11, rtol=0)
    np.testing.assert_allclose(dv, tv.grad.numpy(), atol=1e-11, rtol=0)


def _loss(q, k, v, g, alpha, W):
    table = O.offset_table(alpha, W, round_alpha_to_fp32=False)
    out, _ = O.forward_slab(q, k, v, alpha, W, table=table)
    return float((out * g).sum())


@pytest.mark.parametrize("alpha,W,T", [(0.7317, 4, 64), (1.2913, 6, 300),
                                       (0.9871, 3, 120)])
def test_dalpha_central_difference(alpha, W, T):
    """d(loss)/d(alpha) by central differences in fp64 at an alpha whose
    distances alpha*f stay far from integers, from W and from every i."""
    D = 8
    q, k, v, g = (_rand((T, D), s) for s in (90, 91, 92, 93))
    h = 1e-6
    for f in O.FIB:
        frac = (alpha * f) % 1.0
        assert min(frac, 1 - frac) > 20 * h * f
    table = O.offset_table(alpha, W, round_alpha_to_fp32=False)
    _, _, _, da, _ = O.backward_slab(q, k, v, g, alpha, W, table=table)
    fd = (_loss(q, k, v, g, alpha + h, W) - _loss(q, k, v, g, alpha - h, W)) / (2 * h)
    assert abs(da - fd) <= 1e-6 * max(1.0, abs(fd))


def test_dqkv_central_difference():
    T, D, W, alpha = 90, 4, 4, 0.7317
    q, k, v, g = (_rand((T, D), s) for s in (100, 101, 102, 103))
    dq, dk, dv, _, _ = O.backward_slab(q, k, v, g, alpha, W)
    rng = np.random.default_rng(7)
    h = 1e-6
    for name, x, grad in (("q", q, dq), ("k", k, dk), ("v", v, dv)):
        for _ in range(6):
            i, d = int(rng.integers(T)), int(rng.integers(D))
            xp, xm = x.copy(), x.copy()
            xp[i, d] += h
            xm[i, d] -= h
            args_p = {"q": q, "k": k, "v": v}
            args_m = dict(args_p)
            args_p[name], args_m[name] = xp, xm
            lp = float((O.forward_slab(args_p["q"], args_p["k"], args_p["v"], alpha, W)[0] * g).sum())
            lm = float((O.forward_slab(args_m["q"], args_m["k"], args_m["v"], alpha, W)[0] * g).sum())
            assert abs((lp - lm) / (2 * h) - grad[i, d]) < 1e-7


def test_batched_backward_sums_dalpha():
    B, H, T, D = 2, 2, 80, 8
    q, k, v, g = (_rand((B, H, T, D), s) for s in (110, 111, 112, 113))
    dq, dk, dv, da = O.backward(q, k, v, g, 0.8, 5)
    tot = sum(O.backward_slab(q[b, h], k[b, h], v[b, h], g[b, h], 0.8, 5)[3]
              for b in range(B) for h in range(H))
    assert abs(da - tot) < 1e-9 * max(1, abs(tot))
    assert np.array_equal(dk[1, 0], O.backward_slab(q[1, 0], k[1, 0], v[1, 0], g[1, 0], 0.8, 5)[1])


# ---------------------------------------------------------------- row helpers
def test_row_helpers_match_slabs():
    T, D, W, alpha = 700, 8, 6, 0.6333
    q, k, v, g = (_rand((T, D), s) for s in (120, 121, 122, 123))
    out, lse = O.forward_slab(q, k, v, alpha, W)
    dq, dk, dv, _, _ = O.backward_slab(q, k, v, g, alpha, W)
    rows = np.array([0, 1, 5, 6, 7, 50, 311, 312, 699])
    ro, rl = O.forward_rows(q, k, v, alpha, W, rows)
    np.testing.assert_allclose(ro, out[rows], atol=1e-12, rtol=0)
    np.testing.assert_allclose(rl, lse[rows], atol=1e-12, rtol=0)
    rq, _ = O.dq_rows(q, k, v, g, alpha, W, rows)
    np.testing.assert_allclose(rq, dq[rows], atol=1e-12, rtol=0)
    rk, rv = O.dkdv_rows(q, k, v, g, alpha, W, rows)
    np.testing.assert_allclose(rk, dk[rows], atol=1e-12, rtol=0)
    np.testing.assert_allclose(rv, dv[rows], atol=1e-12, rtol=0)


# ---------------------------------------------------------------- planted mistakes
def _matrix_form_error(monkeypatch=None):
    T, D, W, alpha = 200, 8, 4, float(np.float32(0.7317))
    q, k, v, g = (_rand((T, D), s) for s in (130, 131, 132, 133))
    out, _ = O.forward_slab(q, k, v, alpha, W)
    ref, _ = DF.matrix_form(torch.from_numpy(q), torch.from_numpy(k), torch.from_numpy(v),
                            torch.tensor(alpha, dtype=torch.float64), W)
    return float(np.abs(out - ref.numpy()).max())


def test_pins_catch_swapped_interpolation_weights(monkeypatch):
    orig = O._entry_rows

    def swapped(e, T):
        i0, off, lo, hi = orig(e, T)
        return (i0, off, hi, lo) if e[0] == "tap" else (i0, off, lo, hi)

    monkeypatch.setattr(O, "_entry_rows", swapped)
    assert _matrix_form_error() > 1e-3


def test_pins_catch_off_by_one_window(monkeypatch):
    orig = O._entries
    monkeypatch.setattr(O, "_entries", lambda T, W, tab: orig(T, W + 1, tab))
    assert _matrix_form_error() > 1e-3


def test_pins_catch_wrong_dalpha_sign(monkeypatch):
    T, D, W, alpha = 120, 8, 3, 0.9871
    q, k, v, g = (_rand((T, D), s) for s in (140, 141, 142, 143))
    table = O.offset_table(alpha, W, round_alpha_to_fp32=False)
    h = 1e-6
    fd = (_loss(q, k, v, g, alpha + h, W) - _loss(q, k, v, g, alpha - h, W)) / (2 * h)
    # plant a sign error in the dalpha accumulation only (the table keeps the
    # true distances): the finite-difference pin must reject it
    bad = table._replace(slope=-table.slope)
    _, _, _, da_bad, _ = O.backward_slab(q, k, v, g, alpha, W, table=bad)
    assert abs(da_bad - fd) > 1e-3 * abs(fd)
