"""fsa_backward_noalloc (no workspace argument, nothing allocated; the
library's fixed device scratch serves instead) against fsa_backward with a
caller workspace, through the C ABI: bit for bit (the same kernels run), on
two calls in a row, the second smaller than the first; and the host-side
rejection of a problem beyond the fixed scratch."""

from __future__ import annotations

import ctypes
import os

import numpy as np
import pytest

from static_pattern_sparse_amd import fsa as F
from static_pattern_sparse_amd import inputs as I


def test_beyond_scratch_is_rejected_before_any_device_call():
    """B*H*T rows whose workspace exceeds the fixed array: FSA_ERR_SCRATCH,
    returned from the host checks (the pointers are never dereferenced)."""
    if not os.path.exists(F.LIB_PATH):
        pytest.skip("libfsa.so not built")
    L = F.lib()
    B, H, T, D = 1, 32, 65536, 128
    need = F.fsa_backward_workspace_size(B, H, T, D, F.FSA_DTYPE_BF16)
    assert need > F.FSA_NOALLOC_SCRATCH_BYTES
    fake = ctypes.c_void_p(1 << 20)                    # aligned, never read
    st = L.fsa_backward_noalloc(fake, fake, fake, fake, fake, F.FSA_DTYPE_BF16,
                                B, H, T, D, 1.0, 12, F.FSA_PATTERN_FIB,
                                fake, fake, fake, fake, None)
    assert st == F.FSA_ERR_SCRATCH
    assert "scratch" in L.fsa_status_string(st).decode()
    # the largest long-sequence shape fits
    assert F.fsa_backward_workspace_size(1, 16, 65536, 128, F.FSA_DTYPE_BF16) \
        <= F.FSA_NOALLOC_SCRATCH_BYTES


def _case(torch, B, H, T, D, alpha, W, seed):
    x = I.make_inputs(B, H, T, D, "bf16", 300 + seed, 0)
    q, k, v, g = (I.to_device(x[n], "bf16") for n in ("q", "k", "v", "dout"))
    _, lse = F.fsa_forward(q, k, v, alpha, W)
    ref = F.fsa_backward(q, k, v, g, lse, alpha, W)
    nan = lambda: torch.full((B, H, T, D), float("nan"), device="cuda")
    dq, dk, dv = nan(), nan(), nan()
    da = torch.full((1,), float("nan"), device="cuda")
    F.fsa_backward_noalloc(q, k, v, g, lse, alpha, W, dq, dk, dv, da)
    torch.cuda.synchronize()
    return (dq, dk, dv, da), ref


@pytest.mark.gpu
def test_noalloc_matches_workspace_backward_twice():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    print("[case] noalloc B2 H4 T2000 then B1 H3 T333", flush=True)
    alpha = float(np.float32(0.8333333))
    for B, H, T, D, W, seed in ((2, 4, 2000, 64, 12, 1), (1, 3, 333, 128, 7, 2)):
        got, ref = _case(torch, B, H, T, D, alpha, W, seed)
        for name, a, b in zip(("dq", "dk", "dv", "dalpha"), got, ref):
            assert torch.equal(a, b), name
