"""Pins of the oracle's decoding step (one new query against cached rows).

Source page: Depth-Staggered Fibonacci Spacing for Sparse Attention
(gist.science technical summary): Methodology > Architecture and attention
(the attended set of a query) and Core contributions and results > 2. Learned
dilation is inert (the inference-latency comparison). A decoding query at
position i attends exactly what row i of the full sequence attends, from rows
0..i only. Every test runs on the CPU against independent dense forms
(`tests/dense_forms.py`) or properties.
"""

from __future__ import annotations

import math

import numpy as np
import pytest
import torch

from oracle import fsa_oracle as O
from tests import dense_forms as DF

PATTERNS = [("fib", "lerp"), ("fib", "round"), ("pow2", "lerp"), ("pow2", "round")]


def _rand(shape, seed):
    return np.random.default_rng(seed).standard_normal(shape)


def test_decode_alpha1_equals_dense_row():
    """alpha = 1: the decoding query against rows 0..i equals the last row of
    dense masked attention over the first i + 1 rows (Fibonacci and
    power-of-two sets by enumeration)."""
    D, W = 8, 6
    kc, vc = _rand((1, 1, 700, D), 300), _rand((1, 1, 700, D), 301)
    for base, dists in (("fib", DF.FIB_LIST), ("pow2", DF.POW2_LIST)):
        for i in (0, 3, 5, 6, 12, 13, 54, 55, 233, 699):
            q = _rand((1, 1, D), 302 + i)
            out, lse = O.decode(q, kc, vc, [i], 1.0, W, base=base)
            qs = np.zeros((i + 1, D))
            qs[i] = q[0, 0]
            tq, tk, tv = (torch.from_numpy(x) for x in (qs, kc[0, 0, :i + 1], vc[0, 0, :i + 1]))
            ro, rl = DF.dense_masked(tq, tk, tv, DF.attended_sets(i + 1, W, dists))
            np.testing.assert_allclose(out[0, 0], ro[i].numpy(), atol=1e-12, rtol=0)
            assert abs(lse[0, 0] - float(rl[i])) < 1e-12


@pytest.mark.parametrize("base,mode", PATTERNS)
def test_decode_equals_matrix_form_row(base, mode):
    """Fractional alpha: each decoding query equals row i of the
    interpolation-matrix form (lerp) or of dense masked attention over the
    rounded offsets (round)."""
    D, W, T = 8, 5, 400
    alpha = float(np.float32(0.7317))
    B, H = 3, 2
    kc, vc = _rand((B, H, T, D), 310), _rand((B, H, T, D), 311)
    q = _rand((B, H, D), 312)
    pos = [0, 150, 399]
    out, lse = O.decode(q, kc, vc, pos, alpha, W, base=base, mode=mode)
    tab = O.offset_table(alpha, W, base=base, mode=mode)
    dists = [int(c) for c, k in zip(tab.c, tab.keep) if k]
    for b, i in enumerate(pos):
        for h in range(H):
            qs = np.zeros((i + 1, D))
            qs[i] = q[b, h]
            tq, tk, tv = (torch.from_numpy(x) for x in (qs, kc[b, h, :i + 1], vc[b, h, :i + 1]))
            if mode == "lerp":
                ro, rl = DF.matrix_form(tq, tk, tv, torch.tensor(alpha, dtype=torch.float64),
                                        W, base_list=BASE[base])
            else:
                ro, rl = DF.dense_masked(tq, tk, tv, DF.attended_sets(i + 1, W, dists))
            np.testing.assert_allclose(out[b, h], ro[i].numpy(), atol=1e-12, rtol=0)
            assert abs(lse[b, h] - float(rl[i])) < 1e-12


BASE = {"fib": DF.FIB_LIST, "pow2": DF.POW2_LIST}


@pytest.mark.parametrize("base,mode", PATTERNS)
def test_decode_equals_forward_row(base, mode):
    """The decoding step is the forward pass's row i, for any i."""
    D, W, T = 8, 12, 1100
    alpha = float(np.float32(0.5666667))
    q, k, v = (_rand((T, D), s) for s in (320, 321, 322))
    out, lse = O.forward_slab(q, k, v, alpha, W, base=base, mode=mode)
    rows = [0, 1, 11, 12, 16, 17, 18, 600, 1099]
    qd = np.stack([q[i] for i in rows])[:, None]
    kc = np.broadcast_to(k, (len(rows), 1, T, D))
    vc = np.broadcast_to(v, (len(rows), 1, T, D))
    do, dl = O.decode(qd, kc, vc, rows, alpha, W, base=base, mode=mode)
    np.testing.assert_allclose(do[:, 0], out[rows], atol=1e-12, rtol=0)
    np.testing.assert_allclose(dl[:, 0], lse[rows], atol=1e-12, rtol=0)


def test_decode_reads_no_row_past_its_position():
    """Rows after the query's position (not yet written in a cache) are never
    read: filling them with NaN changes nothing."""
    D, W, T = 8, 4, 300
    kc, vc = _rand((2, 1, T, D), 330), _rand((2, 1, T, D), 331)
    q = _rand((2, 1, D), 332)
    pos = [7, 200]
    out, lse = O.decode(q, kc, vc, pos, 0.9, W)
    kn, vn = kc.copy(), vc.copy()
    for b, i in enumerate(pos):
        kn[b, :, i + 1:] = np.nan
        vn[b, :, i + 1:] = np.nan
    out2, lse2 = O.decode(q, kn, vn, pos, 0.9, W)
    assert np.array_equal(out, out2) and np.array_equal(lse, lse2)


def test_decode_q_zero_counts():
    """Q = 0: lse = ln n_i, with n_i = min(W, i + 1) plus the kept taps that
    reach a row (alpha = 1, W = 8: Fibonacci distances 8, 13, 21, ...)."""
    D, W, T = 4, 8, 1000
    kc, vc = _rand((1, 1, T, D), 340), _rand((1, 1, T, D), 341)
    for i, n in ((0, 1), (7, 8), (8, 9), (13, 10), (100, 14), (987, 19)):
        _, lse = O.decode(np.zeros((1, 1, D)), kc, vc, [i], 1.0, W)
        assert abs(lse[0, 0] - math.log(n)) < 1e-12


def test_decode_rejects_position_outside_cache():
    kc = np.zeros((1, 1, 10, 4))
    with pytest.raises(ValueError):
        O.decode(np.zeros((1, 1, 4)), kc, kc, [10], 1.0, 4)
    with pytest.raises(ValueError):
        O.decode(np.zeros((1, 1, 4)), kc, kc, [-1], 1.0, 4)
