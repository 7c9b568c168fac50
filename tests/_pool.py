"""Process-pool helpers for oracle checks (import only numpy and the oracle)."""

import numpy as np

from oracle import fsa_oracle as O


def slab_dalpha(args):
    q, k, v, g, alpha, W = args
    return O.backward_slab(q, k, v, g, alpha, W)[3]


def slab_check(args):
    """The oracle's forward and backward of one [T, D] slab against the GPU
    results `got` (float32 arrays of that slab): the largest absolute
    difference per output, and the oracle's dalpha of the slab."""
    q, k, v, g, got, alpha, W = args
    q, k, v, g = (x.astype(np.float64) for x in (q, k, v, g))
    ro, rl = O.forward_slab(q, k, v, alpha, W)
    rq, rk, rv, ra, _ = O.backward_slab(q, k, v, g, alpha, W)
    errs = {}
    for name, r in (("out", ro), ("lse", rl), ("dq", rq), ("dk", rk), ("dv", rv)):
        a = got[name]
        errs[name] = float("inf") if not np.isfinite(a).all() else \
            float(np.abs(a.astype(np.float64) - r).max())
    return errs, ra
