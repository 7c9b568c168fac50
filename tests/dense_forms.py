"""Independent dense formulations used to pin the oracle (tests only).

Nothing here is shared with the oracle or with the HIP library. The forms are
deliberately different computations of the same definition
[Depth-Staggered Fibonacci Spacing for Sparse Attention: Methodology >
Architecture and attention > Attended set, Scaling, Implementation]:

* `attended_sets`   -- the attended index set of every query by plain
                       enumeration with Python sets (integer distances only).
* `dense_masked`    -- full T x T score matrix with a boolean mask built from
                       those sets, torch float64, differentiable.
* `matrix_form`     -- every tap as a dense T x T interpolation matrix M_k
                       ((1 - t) on sub-diagonal c_k, t on sub-diagonal c_k - 1),
                       so that the tap's keys are M_k K and its values M_k V;
                       alpha is a torch leaf so autograd yields d/dalpha.
"""

from __future__ import annotations

import math

import torch

FIB_LIST = [1, 2, 3, 5, 8, 13, 21, 34, 55, 89, 144, 233, 377, 610, 987]
# power-of-two control base [same page: Methodology > Control variables]
POW2_LIST = [1 << n for n in range(15)]


def attended_sets(T, window, distances):
    """Per query, the set of key rows it attends (integer distances)."""
    sets = []
    for i in range(T):
        s = {j for j in range(i - window + 1, i + 1) if j >= 0}
        for dist in distances:
            if dist >= window and i - dist >= 0:
                s.add(i - dist)
        sets.append(s)
    return sets


def dense_masked(q, k, v, sets):
    """Masked dense softmax attention; q, k, v torch float64 [T, D]."""
    T, D = q.shape
    mask = torch.zeros(T, T, dtype=torch.bool)
    for i, s in enumerate(sets):
        for j in s:
            mask[i, j] = True
    S = (q @ k.T) / math.sqrt(D)
    S = S.masked_fill(~mask, float("-inf"))
    lse = torch.logsumexp(S, dim=1)
    P = torch.exp(S - lse[:, None])
    return P @ v, lse


def matrix_form(q, k, v, alpha, window, base_list=FIB_LIST):
    """Sparse attention through explicit interpolation matrices.

    alpha: 0-dim float64 torch tensor (may require grad). Distances d = alpha*f
    with f >= ... kept when d >= window; the lower row of query i is
    i - ceil(d), the upper row i - ceil(d) + 1 with weight ceil(d) - d.
    """
    T, D = q.shape
    scale = 1.0 / math.sqrt(D)
    idx = torch.arange(T)
    win_mask = (idx[None, :] <= idx[:, None]) & (idx[None, :] > idx[:, None] - window)
    Sw = (scale * (q @ k.T)).masked_fill(~win_mask, float("-inf"))
    tap_s, tap_v = [], []
    for f in base_list:
        d = alpha * f
        dval = float(d.detach())
        if dval < window:
            continue
        c = math.ceil(dval)
        if c > T - 1:
            continue
        t = c - d
        E_lo = torch.zeros(T, T, dtype=q.dtype)
        E_hi = torch.zeros(T, T, dtype=q.dtype)
        rows = torch.arange(c, T)
        E_lo[rows, rows - c] = 1.0
        E_hi[rows, rows - c + 1] = 1.0
        M = (1.0 - t) * E_lo + t * E_hi
        Kt = M @ k
        Vt = M @ v
        s = scale * (q * Kt).sum(dim=1)
        s = s.masked_fill(idx < c, float("-inf"))
        tap_s.append(s)
        tap_v.append(Vt)
    if tap_s:
        S = torch.cat([Sw, torch.stack(tap_s, dim=1)], dim=1)
    else:
        S = Sw
    lse = torch.logsumexp(S, dim=1)
    P = torch.exp(S - lse[:, None])
    out = P[:, :T] @ v
    for n, Vt in enumerate(tap_v):
        out = out + P[:, T + n, None] * Vt
    return out, lse
