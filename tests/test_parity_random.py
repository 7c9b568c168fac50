"""Seeded random configurations (shape, dtype, alpha, window, pattern) against
the fp64 oracle, forward and backward, through the C ABI.

The draws cover ragged tails (T not a multiple of the 15-query or 14-key
tiles), windows of one to five window blocks (1-69 keys), head dims 64
and 128, both input dtypes and all four tap patterns; a second set draws
sequences of 700-3200 rows, where the longest taps reach back inside the
slab. Tolerances as in test_parity.
"""

from __future__ import annotations

import numpy as np
import pytest

from tests.test_parity import ORACLE_PATTERN, _rand_inputs, _say, check_backward, check_forward

pytestmark = pytest.mark.gpu


def _draw(seed):
    r = np.random.default_rng(1000 + seed)
    B = int(r.integers(1, 3))
    H = int(r.integers(1, 4))
    T = int(r.integers(1, 700))
    D = int(r.choice([64, 128]))
    dtype = "f32" if r.random() < 0.25 else "bf16"
    alpha = float(np.float32(r.uniform(0.5, 1.5)))
    W = int(r.choice([int(r.integers(1, 34)), int(r.integers(34, 60))], p=[0.8, 0.2]))
    pattern = str(r.choice(sorted(ORACLE_PATTERN)))
    return B, H, T, D, dtype, alpha, W, pattern


@pytest.mark.parametrize("seed", range(24))
def test_random_config(seed):
    B, H, T, D, dtype, alpha, W, pattern = _draw(seed)
    _say("random", seed, B, H, T, D, dtype, alpha, W, pattern)
    x = _rand_inputs(B, H, T, D, dtype, seed)
    out, lse = check_forward(x, dtype, alpha, W, pattern)
    check_backward(x, dtype, alpha, W, lse, pattern)


def _draw_long(seed):
    """Longer sequences (700-3200 rows), so that taps up to 1.5 x 987 rows
    back reach rows of the slab."""
    r = np.random.default_rng(50000 + seed)
    B, H = int(r.integers(1, 3)), int(r.integers(1, 3))
    T = int(r.integers(700, 3200))
    D = int(r.choice([64, 128]))
    dtype = "f32" if r.random() < 0.2 else "bf16"
    alpha = float(np.float32(r.uniform(0.5, 1.5)))
    W = int(r.choice([int(r.integers(1, 34)), int(r.integers(34, 70))], p=[0.85, 0.15]))
    pattern = str(r.choice(sorted(ORACLE_PATTERN)))
    return B, H, T, D, dtype, alpha, W, pattern


@pytest.mark.parametrize("seed", range(16))
def test_random_long_config(seed):
    B, H, T, D, dtype, alpha, W, pattern = _draw_long(seed)
    _say("random long", seed, B, H, T, D, dtype, alpha, W, pattern)
    x = _rand_inputs(B, H, T, D, dtype, 7000 + seed)
    out, lse = check_forward(x, dtype, alpha, W, pattern)
    check_backward(x, dtype, alpha, W, lse, pattern)
