"""C-ABI checks that need no GPU: exports, host tables, argument validation.

Only calls that return before any HIP call are made here (host-only entry
points, and compute entry points with arguments the validation rejects).
"""

from __future__ import annotations

import ctypes
import os
import re

import numpy as np
import pytest

from oracle import fsa_oracle as O
from static_pattern_sparse_amd import fsa as F

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "fsa.h")

pytestmark = pytest.mark.skipif(not os.path.exists(F.LIB_PATH),
                                reason="libfsa.so not built")


def _declared():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(fsa_[a-z_0-9]+)\s*\(", text)))


def test_header_declarations_are_exported():
    lib = ctypes.CDLL(F.LIB_PATH)
    names = _declared()
    assert "fsa_forward" in names and "fsa_backward" in names
    for n in names:
        assert hasattr(lib, n), n
    assert set(names) == set(F.EXPORTS)


@pytest.mark.parametrize("kind", [F.FSA_SCHEDULE_FIXED, F.FSA_SCHEDULE_LINEAR,
                                  F.FSA_SCHEDULE_COPRIME])
@pytest.mark.parametrize("L", [1, 2, 5, 16, 17])
def test_schedule_bit_exact_vs_oracle(kind, L):
    if kind == F.FSA_SCHEDULE_COPRIME and np.gcd(7, L) != 1:
        with pytest.raises(F.FsaError):
            F.fsa_schedule(kind, L)
        return
    got = F.fsa_schedule(kind, L)
    ref = O.schedule(kind, L)
    assert np.array_equal(got.view(np.uint32), ref.view(np.uint32))


@pytest.mark.parametrize("alpha", list(O.schedule(O.SCHEDULE_LINEAR, 16)) + [0.7317, 1.2913])
@pytest.mark.parametrize("W", [1, 6, 12, 100])
def test_offsets_vs_oracle(alpha, W):
    c, t, keep = F.fsa_offsets(alpha, W)
    d_r, c_r, t_r, keep_r, _ = O.offset_table(alpha, W)
    assert np.array_equal(c, c_r)
    assert np.array_equal(keep, keep_r)
    assert np.array_equal(t, t_r.astype(np.float32))


def test_schedule_validation():
    with pytest.raises(F.FsaError):
        F.fsa_schedule(F.FSA_SCHEDULE_LINEAR, 0)
    with pytest.raises(F.FsaError):
        F.fsa_schedule(F.FSA_SCHEDULE_LINEAR, 16, alpha_min=0.4)
    with pytest.raises(F.FsaError):
        F.fsa_schedule(F.FSA_SCHEDULE_LINEAR, 16, alpha_min=1.2, alpha_max=1.0)
    with pytest.raises(F.FsaError):
        F.fsa_schedule(F.FSA_SCHEDULE_COPRIME, 16, stride=6)
    with pytest.raises(F.FsaError):
        F.fsa_schedule(9, 16)
    with pytest.raises(F.FsaError):
        F.fsa_offsets(1.6, 8)
    with pytest.raises(F.FsaError):
        F.fsa_offsets(1.0, 0)
    with pytest.raises(F.FsaError):
        F.fsa_offsets(float("nan"), 8)


FAKE = 0x7f0000000000   # never dereferenced: validation fails first


def _fwd(**kw):
    a = dict(q=FAKE, k=FAKE, v=FAKE, dtype=1, B=1, H=1, T=16, D=64, alpha=1.0,
             W=4, out=FAKE, lse=FAKE)
    a.update(kw)
    return F.lib().fsa_forward(*(ctypes.c_void_p(a[n]) if n in ("q", "k", "v", "out", "lse")
                                 else a[n] for n in ("q", "k", "v", "dtype", "B", "H", "T",
                                                     "D", "alpha", "W", "out", "lse")), None)


def test_forward_validation_codes():
    assert _fwd(alpha=1.6) == F.FSA_ERR_INVALID_ARG
    assert _fwd(alpha=0.49) == F.FSA_ERR_INVALID_ARG
    assert _fwd(alpha=float("inf")) == F.FSA_ERR_INVALID_ARG
    assert _fwd(W=0) == F.FSA_ERR_INVALID_ARG
    assert _fwd(T=-1) == F.FSA_ERR_INVALID_ARG
    assert _fwd(D=96) == F.FSA_ERR_UNSUPPORTED
    assert _fwd(D=32) == F.FSA_ERR_UNSUPPORTED
    assert _fwd(dtype=5) == F.FSA_ERR_UNSUPPORTED
    assert _fwd(q=0) == F.FSA_ERR_INVALID_ARG
    assert _fwd(lse=0) == F.FSA_ERR_INVALID_ARG
    assert _fwd(k=FAKE + 2) == F.FSA_ERR_INVALID_ARG       # misaligned
    assert _fwd(B=300, H=300) == F.FSA_ERR_UNSUPPORTED       # too many heads
    assert _fwd(T=1 << 23, D=64) == F.FSA_ERR_UNSUPPORTED    # slab past 32-bit offsets
    assert _fwd(T=1 << 22, D=128) == F.FSA_ERR_UNSUPPORTED
    # an empty problem is a no-op that touches nothing
    assert _fwd(T=0, q=0, k=0, v=0, out=0, lse=0) == F.FSA_OK
    assert _fwd(B=0) == F.FSA_OK


def _bwd(**kw):
    a = dict(q=FAKE, k=FAKE, v=FAKE, g=FAKE, lse=FAKE, dtype=1, B=1, H=1, T=16,
             D=64, alpha=1.0, W=4, dq=FAKE, dk=FAKE, dv=FAKE, da=FAKE, ws=FAKE,
             nbytes=1 << 20)
    a.update(kw)
    ptr = ("q", "k", "v", "g", "lse", "dq", "dk", "dv", "da", "ws")
    order = ("q", "k", "v", "g", "lse", "dtype", "B", "H", "T", "D", "alpha", "W",
             "dq", "dk", "dv", "da", "ws", "nbytes")
    return F.lib().fsa_backward(*(ctypes.c_void_p(a[n]) if n in ptr else a[n]
                                  for n in order), None)


def test_backward_validation_codes():
    assert _bwd(alpha=2.0) == F.FSA_ERR_INVALID_ARG
    assert _bwd(da=0) == F.FSA_ERR_INVALID_ARG
    assert _bwd(g=0) == F.FSA_ERR_INVALID_ARG
    assert _bwd(dv=FAKE + 4) == F.FSA_ERR_INVALID_ARG
    assert _bwd(D=80) == F.FSA_ERR_UNSUPPORTED
    assert _bwd(ws=0) == F.FSA_ERR_WORKSPACE
    assert _bwd(nbytes=16) == F.FSA_ERR_WORKSPACE
    assert _bwd(ws=FAKE + 16) == F.FSA_ERR_WORKSPACE         # not 256-aligned


def test_workspace_size():
    n = F.fsa_backward_workspace_size(8, 8, 1024, 64, F.FSA_DTYPE_BF16)
    assert n >= 8 * 8 * 1024 * 4 and n % 256 == 0
    assert F.fsa_backward_workspace_size(0, 8, 1024, 64, 1) == 0
    assert F.fsa_backward_workspace_size(1, 1, 16, 96, 1) == 0
    big = F.fsa_backward_workspace_size(1, 16, 65536, 128, 1)
    assert big >= 16 * 65536 * 4


# ---------------------------------------------------------------- tap patterns
_ORACLE_PATTERN = {"fib": ("fib", "lerp"), "fib-round": ("fib", "round"),
                   "pow2": ("pow2", "lerp"), "pow2-round": ("pow2", "round")}


@pytest.mark.parametrize("name", sorted(_ORACLE_PATTERN))
@pytest.mark.parametrize("alpha", [0.5, 1.0, 1.5, 0.7317, 0.5666667, 1.2913])
@pytest.mark.parametrize("W", [1, 6, 12])
def test_offsets_ex_vs_oracle(name, alpha, W):
    c, t, keep = F.fsa_offsets(alpha, W, F.PATTERNS[name])
    base, mode = _ORACLE_PATTERN[name]
    tab = O.offset_table(alpha, W, base=base, mode=mode)
    assert np.array_equal(c, tab.c)
    assert np.array_equal(keep, tab.keep)
    assert np.array_equal(t, tab.t.astype(np.float32))


def test_pattern_validation_codes():
    with pytest.raises(F.FsaError):
        F.fsa_offsets(1.0, 8, 8)
    with pytest.raises(F.FsaError):
        F.fsa_offsets(1.0, 8, -1)
    lib = F.lib()
    args = [ctypes.c_void_p(FAKE)] * 3 + [1, 1, 1, 16, 64, 1.0, 4]
    for bad in (8, 16, -1):
        assert lib.fsa_forward_ex(*args, bad, ctypes.c_void_p(FAKE),
                                  ctypes.c_void_p(FAKE), None) == F.FSA_ERR_INVALID_ARG
    bwd = [ctypes.c_void_p(FAKE)] * 5 + [1, 1, 1, 16, 64, 1.0, 4]
    out4 = [ctypes.c_void_p(FAKE)] * 5 + [1 << 20, None]
    assert lib.fsa_backward_ex(*bwd, 8, *out4) == F.FSA_ERR_INVALID_ARG
    assert lib.fsa_backward_dq_ex(*bwd, 8, ctypes.c_void_p(FAKE), ctypes.c_void_p(FAKE),
                                  1 << 20, None) == F.FSA_ERR_INVALID_ARG
    assert lib.fsa_backward_dkdv_ex(*bwd, 8, *out4[1:]) == F.FSA_ERR_INVALID_ARG
    # every valid pattern passes validation up to the first bad argument
    for p in F.PATTERNS.values():
        assert lib.fsa_forward_ex(*args[:-1], 0, p, ctypes.c_void_p(FAKE),
                                  ctypes.c_void_p(FAKE), None) == F.FSA_ERR_INVALID_ARG


def _dec(**kw):
    a = dict(q=FAKE, k=FAKE, v=FAKE, dtype=1, B=2, H=3, T=64, D=64, pos=FAKE,
             alpha=1.0, W=4, pattern=0, out=FAKE, lse=FAKE)
    a.update(kw)
    ptr = ("q", "k", "v", "pos", "out", "lse")
    order = ("q", "k", "v", "dtype", "B", "H", "T", "D", "pos", "alpha", "W",
             "pattern", "out", "lse")
    return F.lib().fsa_decode(*(ctypes.c_void_p(a[n]) if n in ptr else a[n]
                                for n in order), None)


def test_decode_validation_codes():
    assert _dec(alpha=1.6) == F.FSA_ERR_INVALID_ARG
    assert _dec(W=0) == F.FSA_ERR_INVALID_ARG
    assert _dec(T=0) == F.FSA_ERR_INVALID_ARG               # empty cache
    assert _dec(pattern=8) == F.FSA_ERR_INVALID_ARG
    assert _dec(pos=0) == F.FSA_ERR_INVALID_ARG
    assert _dec(pos=FAKE + 2) == F.FSA_ERR_INVALID_ARG      # misaligned int32
    assert _dec(q=FAKE + 8) == F.FSA_ERR_INVALID_ARG
    assert _dec(lse=0) == F.FSA_ERR_INVALID_ARG
    assert _dec(D=96) == F.FSA_ERR_UNSUPPORTED
    assert _dec(dtype=7) == F.FSA_ERR_UNSUPPORTED
    assert _dec(B=300, H=300) == F.FSA_ERR_UNSUPPORTED
    # no query at all is a no-op
    assert _dec(B=0, q=0, k=0, v=0, pos=0, out=0, lse=0) == F.FSA_OK


def test_binding_rejects_mismatched_buffers():
    """The binding checks every caller-supplied tensor against the shape and
    dtype the C call assumes for its pointer (CPU tensors are rejected first)."""
    import torch
    q = torch.zeros(1, 1, 16, 64)
    with pytest.raises(ValueError):
        F.fsa_forward(q, q, q, 1.0, 4)                     # not device tensors
    with pytest.raises(ValueError):
        F._need(torch.zeros(3), (4,), torch.float32, "x")
    with pytest.raises(ValueError):
        F._rows(q, (torch.zeros(1, 1, 15, 64),))


def _rope(**kw):
    a = dict(x=FAKE, din=1, B=2, H=3, T=64, D=64, base=10000.0, pos0=0,
             inverse=0, y=FAKE + 4096, dout=1)
    a.update(kw)
    ptr = ("x", "pos0", "y")
    order = ("x", "din", "B", "H", "T", "D", "base", "pos0", "inverse", "y", "dout")
    return F.lib().fsa_rope(*(ctypes.c_void_p(a[n]) if n in ptr else a[n]
                              for n in order), None)


def test_rope_validation_codes():
    """Argument checks of fsa_rope run before any HIP call (no launch here:
    every call below is rejected, or is the empty no-op)."""
    assert _rope(x=0) == F.FSA_ERR_INVALID_ARG
    assert _rope(y=0) == F.FSA_ERR_INVALID_ARG
    assert _rope(x=FAKE + 8) == F.FSA_ERR_INVALID_ARG       # misaligned rows
    assert _rope(pos0=FAKE + 2) == F.FSA_ERR_INVALID_ARG    # misaligned int32
    assert _rope(D=63) == F.FSA_ERR_INVALID_ARG             # pairs need an even D
    assert _rope(D=0) == F.FSA_ERR_INVALID_ARG
    assert _rope(B=-1) == F.FSA_ERR_INVALID_ARG
    assert _rope(base=1.0) == F.FSA_ERR_INVALID_ARG
    assert _rope(base=float("nan")) == F.FSA_ERR_INVALID_ARG
    assert _rope(base=float("inf")) == F.FSA_ERR_INVALID_ARG
    assert _rope(y=FAKE, din=0, dout=1) == F.FSA_ERR_INVALID_ARG   # in place, two widths
    assert _rope(D=60) == F.FSA_ERR_UNSUPPORTED            # not a multiple of 8
    assert _rope(D=2048) == F.FSA_ERR_UNSUPPORTED
    assert _rope(din=7) == F.FSA_ERR_UNSUPPORTED
    assert _rope(dout=2) == F.FSA_ERR_UNSUPPORTED
    assert _rope(B=65535, H=65535, T=65535) == F.FSA_ERR_UNSUPPORTED   # grid limit
    # no row at all is a no-op
    assert _rope(T=0, x=0, y=0) == F.FSA_OK


def test_rope_binding_checks_buffers():
    import torch
    x = torch.zeros(1, 1, 4, 64)
    with pytest.raises(ValueError):
        F.fsa_rope(x, 10000.0)                              # not a device tensor


def test_learned_alpha_argument_checks():
    """The learned-alpha entry points reject bad arguments before any HIP call
    (fake, never dereferenced pointers where a pointer must be non-null)."""
    L = F.lib()
    fake = ctypes.c_void_p(1 << 20)
    ok = dict(theta_map=F.FSA_THETA_CLAMP, window=12, pattern=F.FSA_PATTERN_FIB)
    inv = F.FSA_ERR_INVALID_ARG
    # layers out of range, bad map, window, pattern (the bf16-out bit is not a tap pattern)
    assert L.fsa_theta_alpha(fake, 0, 0, 12, 0, fake, fake, None) == inv
    assert L.fsa_theta_alpha(fake, 1025, 0, 12, 0, fake, fake, None) == inv
    assert L.fsa_theta_alpha(fake, 4, 7, 12, 0, fake, fake, None) == inv
    assert L.fsa_theta_alpha(fake, 4, 0, 0, 0, fake, fake, None) == inv
    assert L.fsa_theta_alpha(fake, 4, 0, 12, F.FSA_OUT_BF16, fake, fake, None) == inv
    assert L.fsa_theta_alpha(None, 4, 0, 12, 0, fake, fake, None) == inv
    assert L.fsa_theta_alpha(fake, 4, 0, 12, 0, fake, ctypes.c_void_p((1 << 20) + 16), None) == inv
    step = lambda **kw: L.fsa_theta_step(
        kw.get("theta", fake), fake, kw.get("L", 4), kw.get("map", 0), kw.get("opt", 1),
        kw.get("lr", 0.01), kw.get("b1", 0.9), kw.get("b2", 0.999), kw.get("eps", 1e-8),
        kw.get("state", fake), 12, 0, fake, fake, None)
    assert step(opt=2) == inv
    assert step(lr=-1.0) == inv
    assert step(lr=float("nan")) == inv
    assert step(b1=1.0) == inv
    assert step(b2=-0.1) == inv
    assert step(eps=0.0) == inv
    assert step(state=ctypes.c_void_p((1 << 20) + 4)) == inv
    assert step(theta=None) == inv
    del ok
    # device-table attention calls: a table must be given and aligned; the
    # forward's flags take only the bf16-out bit
    q = fake
    assert L.fsa_forward_dev(q, q, q, F.FSA_DTYPE_BF16, 1, 1, 16, 64, None, 12, 0, q, q,
                             None) == inv
    assert L.fsa_forward_dev(q, q, q, F.FSA_DTYPE_BF16, 1, 1, 16, 64, q, 12,
                             F.FSA_MODE_ROUND, q, q, None) == inv
    assert L.fsa_forward_dev(q, q, q, F.FSA_DTYPE_BF16, 1, 1, 16, 96, q, 12, 0, q, q,
                             None) == F.FSA_ERR_UNSUPPORTED
    assert L.fsa_backward_dev(q, q, q, q, q, F.FSA_DTYPE_BF16, 1, 1, 16, 64, None, 12,
                              q, q, q, q, q, 1 << 20, None) == inv
    assert L.fsa_backward_dev(q, q, q, q, q, F.FSA_DTYPE_BF16, 1, 1, 16, 64, q, 12,
                              q, q, q, q, None, 0, None) == F.FSA_ERR_WORKSPACE


def test_fused_rope_argument_checks():
    """fsa_forward_rope / fsa_backward_rope: bf16 rows only (the tile kernels),
    a finite base above 1, an aligned pos0; rejected before any HIP call."""
    L = F.lib()
    p = ctypes.c_void_p(1 << 20)
    bf, f32 = F.FSA_DTYPE_BF16, F.FSA_DTYPE_F32
    fwd = lambda dt=bf, D=64, base=10000.0, pos0=None: L.fsa_forward_rope(
        p, p, p, dt, 1, 1, 16, D, 1.0, 8, 0, base, pos0, p, p, None, None)
    assert fwd(dt=f32) == F.FSA_ERR_UNSUPPORTED
    assert fwd(D=96) == F.FSA_ERR_UNSUPPORTED
    assert fwd(base=1.0) == F.FSA_ERR_INVALID_ARG
    assert fwd(base=float("inf")) == F.FSA_ERR_INVALID_ARG
    assert fwd(pos0=ctypes.c_void_p((1 << 20) + 2)) == F.FSA_ERR_INVALID_ARG
    bwd = lambda dt=bf, base=10000.0: L.fsa_backward_rope(
        p, p, p, p, p, dt, 1, 1, 16, 64, 1.0, 8, 0, base, None, p, p, p, p, p, 1 << 20, None)
    assert bwd(dt=f32) == F.FSA_ERR_UNSUPPORTED
    assert bwd(base=0.5) == F.FSA_ERR_INVALID_ARG
