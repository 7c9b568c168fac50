"""The library's calls inside a HIP graph (torch.cuda.CUDAGraph on ROCm).

The entry points allocate nothing, never synchronise and launch only on the
stream they are given, so a caller can capture them. The graph here holds a
forward, the two backward stages, a decoding step and RoPE passes (forward and
inverse, with device start positions); it is replayed several
times, with eager work and synchronisations in between, and every replay must
reproduce the eager results bit for bit.
"""

from __future__ import annotations

import ctypes

import numpy as np
import pytest

from static_pattern_sparse_amd import inputs as I

pytestmark = pytest.mark.gpu


def test_captured_calls_replay_exactly():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from static_pattern_sparse_amd import fsa as F
    print("[case] graph capture and replay", flush=True)
    B, H, T, D, W, alpha = 2, 2, 700, 64, 12, float(np.float32(0.8))
    x = I.make_inputs(B, H, T, D, "bf16", 85, 0)
    q, k, v, g = (I.to_device(x[n], "bf16") for n in ("q", "k", "v", "dout"))
    dx = I.make_decode_inputs(B, H, T, D, "bf16", 86, 0, [699, 350])
    dq_, dk_, dv_ = (I.to_device(dx[n], "bf16") for n in ("q", "k", "v"))
    pos = torch.from_numpy(dx["pos"]).to("cuda")

    def bufs():
        f = lambda *s: torch.full(s, float("nan"), device="cuda")
        return dict(out=f(B, H, T, D), lse=f(B, H, T), dq=f(B, H, T, D), dk=f(B, H, T, D),
                    dv=f(B, H, T, D), da=f(1), dout=f(B, H, D), dlse=f(B, H),
                    qr=f(B, H, T, D).to(torch.bfloat16), dqp=f(B, H, T, D))

    ws = torch.empty(F.fsa_backward_workspace_size(B, H, T, D, F.FSA_DTYPE_BF16),
                     dtype=torch.uint8, device="cuda")

    def run(o, stream):
        F.fsa_forward(q, k, v, alpha, W, out=o["out"], lse=o["lse"], stream=stream)
        F.fsa_backward_dq(q, k, v, g, o["lse"], alpha, W, o["dq"], ws, stream=stream)
        F.fsa_backward_dkdv(q, k, v, g, o["lse"], alpha, W, o["dk"], o["dv"], o["da"], ws,
                            stream=stream)
        F.fsa_decode(dq_, dk_, dv_, pos, alpha, W, out=o["dout"], lse=o["dlse"], stream=stream)
        F.fsa_rope(q, 10000.0, pos, out=o["qr"], stream=stream)
        F.fsa_rope(o["dq"], 10000.0, pos, inverse=True, out=o["dqp"], stream=stream)

    ref = bufs()
    run(ref, None)
    torch.cuda.synchronize()

    got = bufs()
    s = torch.cuda.Stream()
    graph = torch.cuda.CUDAGraph()
    torch.cuda.synchronize()
    with torch.cuda.graph(graph, stream=s):
        run(got, s)
    for rep in range(3):
        for t in got.values():
            t.fill_(float("nan"))                 # eager work between replays
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for name in ref:
            assert torch.equal(got[name], ref[name]), f"replay {rep}: {name}"
