"""Pins of the oracle's RoPE pass (oracle.rope, reading R12) that do not
restate its formula: the complex-number form of the rotation, hand values,
the group laws of rotations, the adjoint (transpose) property that makes the
inverse the gradient map, and the relative-position property that the page's
length-extrapolation argument rests on [DSFS: Core contributions and results
> 3. Length extrapolation, mechanism: a fixed offset sees the same RoPE
angle at every position].
"""

from __future__ import annotations

import math

import numpy as np
import pytest

from oracle import fsa_oracle as O
from static_pattern_sparse_amd import inputs as I


def _x(shape, seed):
    return np.random.default_rng(seed).standard_normal(shape)


def test_complex_form():
    """Each pair (x[m], x[m + D/2]) is the complex number x[m] + i x[m + D/2]
    multiplied by exp(i * position * base^(-2m/D))."""
    B, H, T, D, base = 2, 3, 17, 24, 10000.0
    x = _x((B, H, T, D), 1)
    pos0 = np.array([5, 40000])
    y = O.rope(x, base, pos0)
    half = D // 2
    z = x[..., :half] + 1j * x[..., half:]
    for b in range(B):
        for m in range(half):
            freq = math.exp(-2.0 * m / D * math.log(base))
            rot = np.exp(1j * (pos0[b] + np.arange(T)) * freq)
            w = z[b, :, :, m] * rot[None, :]
            assert np.allclose(y[b, :, :, m], w.real, rtol=0, atol=1e-10)
            assert np.allclose(y[b, :, :, half + m], w.imag, rtol=0, atol=1e-10)


def test_hand_values():
    """D = 2: the one pair turns by the position in radians for any base.
    D = 4, base 100: pair 0 turns by p, pair 1 by p / 10."""
    x = np.array([1.0, 0.0]).reshape(1, 1, 1, 2)
    for p in (0, 1, 3, 1000):
        y = O.rope(x, 10000.0, [p])[0, 0, 0]
        assert y[0] == pytest.approx(math.cos(p), abs=1e-14)
        assert y[1] == pytest.approx(math.sin(p), abs=1e-14)
    x = np.array([0.0, 0.0, 0.0, 1.0]).reshape(1, 1, 1, 4)   # pair 1, imaginary part
    y = O.rope(x, 100.0, [10])[0, 0, 0]
    assert y == pytest.approx([0.0, -math.sin(1.0), 0.0, math.cos(1.0)], abs=1e-14)


def test_position_zero_is_identity():
    x = _x((1, 2, 1, 64), 2)
    assert np.array_equal(O.rope(x, 10000.0, [0]), x)


def test_angles_add():
    """Rotating a row at position a and then at position b equals one rotation
    at a + b (single-row slabs, so the row offset t is 0)."""
    x = _x((3, 2, 1, 32), 3)
    a, b = np.array([7, 1000, 65535]), np.array([2, 31, 4096])
    assert np.allclose(O.rope(O.rope(x, 500000.0, a), 500000.0, b),
                       O.rope(x, 500000.0, a + b), rtol=0, atol=1e-11)


def test_inverse_undoes_and_is_the_transpose():
    """inverse(rope(x)) = x, and <rope(x), g> = <x, rope(g, inverse)> for all
    x, g: the inverse is the adjoint, so it carries the gradient with respect
    to rotated rows back to the rows before rotation."""
    x, g = _x((2, 2, 9, 16), 4), _x((2, 2, 9, 16), 5)
    pos0 = np.array([3, 12345])
    y = O.rope(x, 10000.0, pos0)
    assert np.allclose(O.rope(y, 10000.0, pos0, inverse=True), x, rtol=0, atol=1e-12)
    lhs = float((y * g).sum())
    rhs = float((x * O.rope(g, 10000.0, pos0, inverse=True)).sum())
    assert lhs == pytest.approx(rhs, rel=1e-12)


def test_pair_norms_kept():
    x = _x((1, 3, 11, 64), 6)
    y = O.rope(x, 10000.0, [777])
    nx = x[..., :32] ** 2 + x[..., 32:] ** 2
    ny = y[..., :32] ** 2 + y[..., 32:] ** 2
    assert np.allclose(nx, ny, rtol=1e-12, atol=0)


def test_scores_depend_on_offset_only():
    """rope(q at i) . rope(k at j) = q . rope(k at j - i): a tap at a fixed
    distance meets the same rotation at every query position."""
    D, base = 64, 10000.0
    q, k = _x((1, 1, 1, D), 7), _x((1, 1, 1, D), 8)
    for i, j in ((100, 13), (4000, 3013), (65000, 64013), (5, 5)):
        lhs = float((O.rope(q, base, [i]) * O.rope(k, base, [j])).sum())
        rhs = float((q * O.rope(k, base, [j - i])).sum())
        assert lhs == pytest.approx(rhs, abs=1e-9)
    # the same offset at two positions gives the same score
    s1 = float((O.rope(q, base, [200]) * O.rope(k, base, [200 - 89])).sum())
    s2 = float((O.rope(q, base, [3000]) * O.rope(k, base, [3000 - 89])).sum())
    assert s1 == pytest.approx(s2, abs=1e-9)


def test_rows_follow_positions():
    """Row t of a slab equals the single row rotated at pos0 + t."""
    x = _x((2, 1, 6, 8), 9)
    pos0 = np.array([0, 50])
    y = O.rope(x, 10000.0, pos0)
    for b in range(2):
        for t in range(6):
            yt = O.rope(x[b:b + 1, :, t:t + 1], 10000.0, [pos0[b] + t])
            assert np.array_equal(yt[0, :, 0], y[b, :, t])


def test_same_rotation_as_the_generator():
    """The attention inputs come from the generator's RoPE: the oracle's pass
    agrees with it on the same fp64 rows (one convention across the tests)."""
    T, D = 300, 64
    x = _x((T, D), 10)
    cos, sin = I.rope_tables(T, D, 10000.0)
    gen = I._rope(x, cos, sin)
    assert np.allclose(O.rope(x[None, None], 10000.0)[0, 0], gen, rtol=0, atol=1e-12)
