"""Process-pool helper for oracle sums (imports only numpy and the oracle)."""

from oracle import fsa_oracle as O


def slab_dalpha(args):
    q, k, v, g, alpha, W = args
    return O.backward_slab(q, k, v, g, alpha, W)[3]
