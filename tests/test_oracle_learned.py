"""Pins of the oracle's learned-alpha step (reading R16): the map from theta
to alpha and its slope, and the optimizer update.

* central differences in theta of the chained loss sum_l <dout_l, out_l>,
  with alpha_l = alpha(theta_l) in fp64, against dL/dalpha (the oracle's
  backward) times the map's slope, for both maps and at the clip's flat part;
* hand-worked updates (tests/golden/learned_steps.txt);
* the map's invariants (alpha = 1 at the initial theta, range, symmetry);
* a planted slope error is caught.
[Depth-Staggered Fibonacci Spacing for Sparse Attention: Methodology >
Experimental variables, Learned; Architecture and attention > Scaling]
"""

from __future__ import annotations

import math
import os

import numpy as np
import pytest

from oracle import fsa_oracle as O

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "learned_steps.txt")


def _slabs(L, T=64, D=8, seed=5):
    r = np.random.default_rng(seed)
    return [tuple(r.standard_normal((T, D)) for _ in range(4)) for _ in range(L)]


def _loss(slabs, thetas, theta_map, W):
    tot = 0.0
    for (q, k, v, g), th in zip(slabs, thetas):
        a = O.theta_to_alpha(th, theta_map)
        tab = O.offset_table(a, W, round_alpha_to_fp32=False)
        out, _ = O.forward_slab(q, k, v, a, W, table=tab)
        tot += float((g * out).sum())
    return tot


def _chain_grad(slabs, thetas, theta_map, W):
    """g_l = dL/dalpha_l (oracle backward at the fp64 alpha) * dalpha/dtheta."""
    da = []
    for (q, k, v, g), th in zip(slabs, thetas):
        a = O.theta_to_alpha(th, theta_map)
        tab = O.offset_table(a, W, round_alpha_to_fp32=False)
        da.append(O.backward_slab(q, k, v, g, a, W, table=tab)[3])
    _, _, _, grad = O.theta_step(thetas, da, [0.0] * len(thetas), [0.0] * len(thetas),
                                 0, theta_map, O.OPT_SGD, 0.0)
    return grad


def _away_from_kinks(theta, theta_map, W, h):
    """alpha*f_k at least 20 h f_k from an integer and from W for every k."""
    a = O.theta_to_alpha(theta, theta_map)
    da = h * max(O.dalpha_dtheta(theta, theta_map), 1e-12)
    for f in O.FIB:
        d = a * f
        if abs(d - round(d)) < 20 * da * f + 1e-9 or abs(d - W) < 20 * da * f:
            return False
    return True


@pytest.mark.parametrize("theta_map,thetas", [
    (O.THETA_CLAMP, [0.7317, 1.2913, 0.9411]),
    (O.THETA_TANH, [0.3101, -0.7207, 0.0517]),
])
def test_theta_gradient_matches_central_differences(theta_map, thetas):
    W, h = 4, 1e-6
    for th in thetas:
        assert _away_from_kinks(th, theta_map, W, h)
    slabs = _slabs(len(thetas))
    grad = _chain_grad(slabs, thetas, theta_map, W)
    for l in range(len(thetas)):
        tp, tm = list(thetas), list(thetas)
        tp[l] += h
        tm[l] -= h
        fd = (_loss(slabs, tp, theta_map, W) - _loss(slabs, tm, theta_map, W)) / (2 * h)
        assert abs(fd - grad[l]) <= 1e-6 * max(1.0, abs(fd)), (l, fd, grad[l])
        assert abs(grad[l]) > 1e-3            # a non-trivial gradient


def test_clip_is_flat_outside_the_range():
    """theta past 1.5 (or below 0.5) gives alpha at the bound: the loss does not
    move with theta there, and the chained gradient is 0."""
    slabs = _slabs(2, seed=9)
    thetas = [1.73, 0.21]
    grad = _chain_grad(slabs, thetas, O.THETA_CLAMP, 4)
    assert list(grad) == [0.0, 0.0]
    for l in range(2):
        tp = list(thetas)
        tp[l] += 1e-3
        assert _loss(slabs, tp, O.THETA_CLAMP, 4) == _loss(slabs, thetas, O.THETA_CLAMP, 4)


def _golden():
    rows = []
    for line in open(GOLDEN):
        line = line.split("#")[0].strip()
        if not line:
            continue
        lhs, rhs = line.split("->")
        a = lhs.split()
        rows.append((a[0], a[1], [float(x) for x in a[2:]], [float(x) for x in rhs.split()]))
    return rows


MAPS = {"clamp": O.THETA_CLAMP, "tanh": O.THETA_TANH}
OPTS = {"sgd": O.OPT_SGD, "adam": O.OPT_ADAM}


@pytest.mark.parametrize("row", _golden(), ids=lambda r: f"{r[0]}-{r[1]}")
def test_hand_worked_updates(row):
    mp, opt, vals, want = row
    lr, b1, b2, eps, step, theta, dalpha, m, v = vals
    th, m2, v2, g = O.theta_step([theta], [dalpha], [m], [v], int(step), MAPS[mp],
                                 OPTS[opt], lr, b1, b2, eps)
    for got, exp in zip((th[0], m2[0], v2[0], g[0]), want):
        assert abs(got - exp) <= 1e-15 * max(1.0, abs(exp)) + 1e-17, (got, exp)


def test_constant_gradient_adam_moves_lr_per_step():
    """With a constant gradient the bias-corrected moments are g and g^2 at
    every step, so each Adam step moves theta by lr * |g| / (|g| + eps)."""
    th, m, v = [1.2], [0.0], [0.0]
    for s in range(6):
        new, m, v, _ = O.theta_step(th, [-0.5], m, v, s, O.THETA_TANH, O.OPT_ADAM, 0.003)
        g = -0.5 * O.dalpha_dtheta(th[0], O.THETA_TANH)
        # the slope changes with theta, so the moments see a slowly varying g;
        # the move stays within 1% of lr
        assert abs((new[0] - th[0]) - 0.003) < 3e-5, (s, new[0] - th[0], g)
        th = list(new)


def test_map_invariants():
    for mp in (O.THETA_CLAMP, O.THETA_TANH):
        assert O.alpha_of_theta(O.theta_init(mp), mp) == 1.0
    for t in np.linspace(-6, 6, 97):
        a = O.theta_to_alpha(t, O.THETA_TANH)
        assert 0.5 <= a <= 1.5
        assert abs((a - 1.0) + (O.theta_to_alpha(-t, O.THETA_TANH) - 1.0)) < 1e-15
        assert O.theta_to_alpha(t, O.THETA_CLAMP) == min(max(t, 0.5), 1.5)
    assert O.dalpha_dtheta(0.0, O.THETA_TANH) == 0.5
    assert O.dalpha_dtheta(0.5, O.THETA_CLAMP) == 1.0
    assert O.dalpha_dtheta(1.5, O.THETA_CLAMP) == 1.0
    assert O.dalpha_dtheta(1.5000001, O.THETA_CLAMP) == 0.0
    # the fp32 alpha is the fp64 map rounded once
    assert O.alpha_of_theta(0.3, O.THETA_TANH) == float(np.float32(1 + 0.5 * math.tanh(0.3)))


def test_planted_slope_error_is_caught(monkeypatch):
    """A tanh slope without the factor 1/2 fails the central-difference pin."""
    good = O.dalpha_dtheta
    monkeypatch.setattr(O, "dalpha_dtheta",
                        lambda t, mp: 2.0 * good(t, mp) if mp == O.THETA_TANH else good(t, mp))
    with pytest.raises(AssertionError):
        test_theta_gradient_matches_central_differences(O.THETA_TANH, [0.3101])
