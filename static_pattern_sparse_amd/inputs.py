"""Seeded synthetic inputs for Fibonacci-spaced sparse attention.

This module only makes inputs. It holds none of the attention arithmetic, so
the HIP path and the CPU checker can both consume what it returns.

Recipe (the same for every workload):

* q, k, v and the upstream gradient dout are i.i.d. N(0, 1), drawn in float64
  from numpy's PCG64 seeded with SeedSequence([seed_root, workload_id, layer,
  tensor_id]) with tensor_id q=0, k=1, v=2, dout=3, one (b, h) slab after the
  other in row-major [B, H, T, D] order; seed_root is 20260630 unless a caller
  asks for another draw.
* q and k are then rotated by RoPE at positions 0..T-1 ("rotate-half" pairing
  (m, m + D/2), angle p * base**(-2m/D)), still in float64: the attention
  layer applies RoPE before its gather [Depth-Staggered Fibonacci Spacing for
  Sparse Attention: Methodology > Architecture and attention > Implementation],
  so the attention inputs are post-RoPE rows. Unscaled ("native") RoPE, as in
  the page's Significance section; bases 10000, or 500000 for the 65536-token
  workload.
* Each value is rounded once to the storage dtype, round-to-nearest-even:
  float64 -> float32, and for bf16 further float32 -> bf16.

Workloads (shapes of the page's 16-layer, 512-wide model: 8 heads x 64, trained
at 1024 tokens and evaluated at 4096 [Methodology; Core results section 3]):
see WORKLOADS.
"""

from __future__ import annotations

import dataclasses

import numpy as np

SEED_ROOT = 20260630
TENSOR_IDS = {"q": 0, "k": 1, "v": 2, "dout": 3}


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    workload_id: int
    B: int
    H: int
    T: int
    D: int
    dtype: str          # "f32" or "bf16"
    schedule: str       # "fixed", "linear" or "coprime"
    windows: tuple
    layers: int
    rope_base: float
    backward: bool


WORKLOADS = {w.name: w for w in [
    Workload("fixed_f32_b1h4t256d64_w8", 1, 1, 4, 256, 64, "f32", "fixed",
             (8,), 1, 10000.0, False),
    Workload("linear16_bf16_b8h8t1024d64_w12", 2, 8, 8, 1024, 64, "bf16",
             "linear", (12,), 16, 10000.0, False),
    Workload("coprime16_bf16_b4h8t4096d64_w6-12", 3, 4, 8, 4096, 64, "bf16",
             "coprime", (6, 8, 10, 12), 16, 10000.0, False),
    Workload("linear16_bwd_bf16_b8h8t1024d64_w12", 4, 8, 8, 1024, 64, "bf16",
             "linear", (12,), 16, 10000.0, True),
    Workload("linear16_bf16_b1h16t65536d128_w12", 5, 1, 16, 65536, 128,
             "bf16", "linear", (12,), 16, 500000.0, True),
    # decoding step: one query per (b, h) against caches of 4096 rows (the
    # evaluation length); four distinct layer caches serve the 16 layers
    Workload("decode16_bf16_b8h8t4096d64_w12", 6, 8, 8, 4096, 64, "bf16",
             "linear", (12,), 16, 10000.0, False),
]}
DECODE_CACHES = 4


def _rng(workload_id: int, layer: int, tensor: str,
         seed_root: int = SEED_ROOT) -> np.random.Generator:
    ss = np.random.SeedSequence([int(seed_root), int(workload_id), int(layer),
                                 TENSOR_IDS[tensor]])
    return np.random.Generator(np.random.PCG64(ss))


def round_to_bf16(x: np.ndarray) -> np.ndarray:
    """float32 -> nearest-even bf16 value, returned as float32 (exact)."""
    x32 = np.ascontiguousarray(x, dtype=np.float32)
    u = x32.view(np.uint32).astype(np.uint64)
    u = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return (u.astype(np.uint32) << 16).view(np.float32)


def bf16_bits(x: np.ndarray) -> np.ndarray:
    """Upper 16 bits of float32 values that are already exact bf16 values."""
    x32 = np.ascontiguousarray(x, dtype=np.float32)
    return (x32.view(np.uint32) >> 16).astype(np.uint16)


def rope_tables(T: int, D: int, base: float):
    half = D // 2
    inv = base ** (-2.0 * np.arange(half, dtype=np.float64) / D)
    ang = np.arange(T, dtype=np.float64)[:, None] * inv[None, :]
    return np.cos(ang), np.sin(ang)


def _rope(x: np.ndarray, cos: np.ndarray, sin: np.ndarray) -> np.ndarray:
    half = x.shape[-1] // 2
    a, b = x[..., :half], x[..., half:]
    return np.concatenate([a * cos - b * sin, b * cos + a * sin], axis=-1)


def make_tensor(B, H, T, D, dtype, workload_id, layer, tensor, rope_base=None,
                seed_root=SEED_ROOT):
    """One input tensor [B, H, T, D] as float32 holding dtype-exact values."""
    rng = _rng(workload_id, layer, tensor, seed_root)
    out = np.empty((B, H, T, D), dtype=np.float32)
    tabs = rope_tables(T, D, rope_base) if rope_base is not None else None
    for b in range(B):
        for h in range(H):
            x = rng.standard_normal((T, D))
            if tabs is not None:
                x = _rope(x, *tabs)
            x32 = x.astype(np.float32)
            out[b, h] = round_to_bf16(x32) if dtype == "bf16" else x32
    return out


def make_inputs(B, H, T, D, dtype, workload_id, layer, rope_base=10000.0,
                with_dout=True, seed_root=SEED_ROOT):
    """q, k (post-RoPE), v and optionally dout for one layer."""
    res = {}
    for name in ("q", "k", "v") + (("dout",) if with_dout else ()):
        base = rope_base if name in ("q", "k") else None
        res[name] = make_tensor(B, H, T, D, dtype, workload_id, layer, name,
                                base, seed_root)
    return res


def workload_inputs(w: Workload, layer: int, with_dout=None, seed_root=SEED_ROOT):
    if with_dout is None:
        with_dout = True
    return make_inputs(w.B, w.H, w.T, w.D, w.dtype, w.workload_id, layer,
                       w.rope_base, with_dout, seed_root)


def to_device(x: np.ndarray, dtype: str, device="cuda"):
    """Upload a dtype-exact float32 array as a torch tensor of that dtype."""
    import torch
    if dtype == "bf16":
        bits = bf16_bits(x).view(np.int16)
        return torch.from_numpy(bits).view(torch.bfloat16).to(device)
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(device)


def decode_positions(B: int, T: int) -> np.ndarray:
    """Query position per batch entry of a decoding step: the last row of the
    cache for entry 0, then 61 rows earlier per entry (sequences of different
    lengths in one batch)."""
    return np.array([max(0, T - 1 - 61 * b) for b in range(B)], dtype=np.int32)


def make_decode_inputs(B, H, T, D, dtype, workload_id, layer, positions,
                       rope_base=10000.0):
    """One decoding step: caches k, v [B, H, T, D] (k post-RoPE at positions
    0..T-1, as make_tensor), queries q [B, H, D] drawn N(0, 1) and rotated to
    position pos[b] (tensor id of q), and pos [B] int32."""
    pos = np.asarray(positions, dtype=np.int32)
    k = make_tensor(B, H, T, D, dtype, workload_id, layer, "k", rope_base)
    v = make_tensor(B, H, T, D, dtype, workload_id, layer, "v", None)
    cos, sin = rope_tables(T, D, rope_base)
    rng = _rng(workload_id, layer, "q")
    q = np.empty((B, H, D), dtype=np.float32)
    for b in range(B):
        x = _rope(rng.standard_normal((H, D)), cos[pos[b]], sin[pos[b]])
        x32 = x.astype(np.float32)
        q[b] = round_to_bf16(x32) if dtype == "bf16" else x32
    return {"q": q, "k": k, "v": v, "pos": pos}


def decode_inputs(w: Workload, layer: int):
    """The decoding workload's inputs for one layer (caches cycle over
    DECODE_CACHES layers)."""
    return make_decode_inputs(w.B, w.H, w.T, w.D, w.dtype, w.workload_id,
                              layer % DECODE_CACHES, decode_positions(w.B, w.T),
                              w.rope_base)
