#!/usr/bin/env python3
"""Fibonacci-spaced sparse attention: forward + backward throughput on one MI355X.

One step = forward (out, lse) and backward (dq, dk, dv, dalpha) of every layer
of a 16-layer linear-stagger stack, B=8, H=8, T=1024, D=64, W=12, bf16 inputs
(the page's 16-layer, 8x64-wide model at its 1024-token training length;
Depth-Staggered Fibonacci Spacing for Sparse Attention, Methodology). Each
layer has its own input and output buffers (about 1.5 GiB in all, more than the
256 MB Infinity Cache), so a layer's data is not cached from one step to the
next. Inputs are seeded N(0,1) synthetic tensors (post-RoPE q, k) and sit in
HBM before the timed region starts.

A step runs the forward of every layer in layer order, then the backward of
every layer in reverse order, each as its two stages (dq, Delta and dalpha
partials; then dk, dv and dalpha); each layer has its own backward workspace.
ms_per_step and value come from the host clock around the timed steps, with no
event between launches. The per-kernel times come from a second pass over as
many steps with a HIP event before every launch, recorded on the launch
stream. Those events are created without the system-scope fence that a default
event record issues: that fence writes back and invalidates the caches and
slows the launch that follows.

value = layers * B * H * T / step time (token-heads per second, every layer
counted). The JSON line also carries:
  pass_tokens_heads_per_s  the forward and the backward (both stages) each
                as B*H*T over its event-timed mean per layer;
  copy_gbs      a plain 1 GiB device copy's read+write GB/s, for context;
  roofline      the dominant kernel's algorithmic bytes per launch divided by
                its mean event-to-event launch time, against the 8 TB/s HBM
                peak; traffic from committed rocprofv3 counter summaries when
                they match the current kernel source, else null;
  cpu_baseline  the fp64 oracle on the host cores over the same step;
  t4096         the same step at B=4, H=8, T=4096, coprime schedule, W=12, and
                the forward over the window sweep W = 6, 8, 10, 12;
  t65536        one layer (forward and backward) at B=1, H=16, T=65536, D=128;
  decode        a decoding step (one new query per (b, h) in each of the 16
                layers, B=8, H=8, caches of 4096 rows, W=12): time per step,
                tokens per second and the mean launch time, and the step time
                with its 16 launches captured once in a HIP graph and replayed.
                Four distinct layer caches serve the 16 layers in turn;
  rope          the RoPE pass at the training size (B=8, H=8, T=1024, D=64,
                base 10000; q and k of every layer) and at B=1, H=16,
                T=65536, D=128 (base 500000): pre-RoPE rows into bf16 rows,
                and fp32 gradients turned back; mean launch time and GB/s
                over the algorithmic bytes (each element read and written
                once). Not part of the step: the attention step takes
                post-RoPE inputs.

    python bench.py [--steps K] [--warmup W] [--gpus 1]
"""

from __future__ import annotations

import argparse
import hashlib
import json
import math
import multiprocessing
import os
import re
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
METRIC = "Fib-sparse attn fwd+bwd tokens·heads/s and % peak HBM GB/s at T=1024/4096"
PROFILES = os.path.join(ROOT, "profiles")
KERNEL_SOURCES = [os.path.join(ROOT, "static_pattern_sparse_amd", "csrc", n)
                  for n in ("fsa_vec.hip", "fsa_mfma.hip")]


def stage_bytes(D, in_bytes, out_bytes=4):
    """Algorithmic HBM bytes per token-head of every kernel: each tensor the
    kernel must read or write, once."""
    row_in = D * in_bytes
    return {
        "fwd": 3 * row_in + out_bytes * D + 4,         # q k v -> out lse
        "bwd_dq": 4 * row_in + 4 + 4 * D + 4,          # q k v dout lse -> dq delta
        "bwd_dkdv": 4 * row_in + 8 + 8 * D,            # q k v dout lse delta -> dk dv dalpha
    }


def algo_bytes(D, in_bytes, out_bytes=4):
    """Algorithmic bytes per token-head of the forward and of the backward as
    a whole (each input read once, each output written once)."""
    row_in = D * in_bytes
    return {"fwd": 3 * row_in + out_bytes * D + 4,
            "bwd": 4 * row_in + 4 + 12 * D}


class Stack:
    """Device buffers of every layer of one workload."""

    def __init__(self, wl, window, layers, torch, F, I, pattern="fib", out_bf16=False,
                 seed_root=None):
        self.torch, self.F = torch, F
        self.wl, self.W, self.layers = wl, window, layers
        self.pattern = F.PATTERNS[pattern]
        self.out_bytes = 2 if out_bf16 else 4
        out_dt = torch.bfloat16 if out_bf16 else torch.float32
        kind = {"linear": F.FSA_SCHEDULE_LINEAR, "coprime": F.FSA_SCHEDULE_COPRIME,
                "fixed": F.FSA_SCHEDULE_FIXED}[wl.schedule]
        self.alphas = F.fsa_schedule(kind, wl.layers)
        B, H, T, D = wl.B, wl.H, wl.T, wl.D
        dev = "cuda"
        self.L = []
        self.host = []                 # the layers' host inputs (oracle checks)
        dt = F.FSA_DTYPE_BF16 if wl.dtype == "bf16" else F.FSA_DTYPE_F32
        ws_bytes = F.fsa_backward_workspace_size(B, H, T, D, dt)
        seed = I.SEED_ROOT if seed_root is None else seed_root
        for l in range(layers):
            x = I.workload_inputs(wl, l, seed_root=seed)
            self.host.append(x)
            t = {n: I.to_device(x[n], wl.dtype) for n in ("q", "k", "v", "dout")}
            f32 = lambda *s: torch.empty(s, dtype=torch.float32, device=dev)
            t.update(out=torch.empty((B, H, T, D), dtype=out_dt, device=dev),
                     lse=f32(B, H, T), dq=f32(B, H, T, D),
                     dk=f32(B, H, T, D), dv=f32(B, H, T, D), dalpha=f32(1),
                     ws=torch.empty(max(ws_bytes, 1), dtype=torch.uint8, device=dev))
            self.L.append(t)
        self._prepare_calls(torch, F)

    def snapshot(self, check_layers):
        """What the oracle checks need once the device buffers are freed: the
        host inputs, the alphas and the GPU results of `check_layers`."""
        import types
        return types.SimpleNamespace(
            wl=self.wl, layers=self.layers, W=self.W, alphas=self.alphas,
            out_bytes=self.out_bytes, host=self.host,
            got={l: self.results(l) for l in check_layers},
            da={l: self.dalpha(l) for l in check_layers})

    def results(self, l):
        """Layer l's GPU results as host float32 arrays."""
        t = self.L[l]
        return {n: t[n].float().cpu().numpy() for n in ("out", "lse", "dq", "dk", "dv")}

    def dalpha(self, l):
        return float(self.L[l]["dalpha"].item())

    def _prepare_calls(self, torch, F):
        """Pre-marshal every launch of a step (raw ctypes argument tuples), so
        the host enqueues far faster than the GPU drains."""
        import ctypes
        lib = F.lib()
        vp, f32 = ctypes.c_void_p, ctypes.c_float
        wl = self.wl
        B, H, T, D = wl.B, wl.H, wl.T, wl.D
        dt = F.FSA_DTYPE_BF16 if wl.dtype == "bf16" else F.FSA_DTYPE_F32
        stream = vp(torch.cuda.current_stream().cuda_stream)
        fwd, dq, dkdv = [], [], []
        for l, t in enumerate(self.L):
            p = {n: vp(x.data_ptr()) for n, x in t.items()}
            nws = t["ws"].numel()
            a = f32(float(self.alphas[l]))
            pt = self.pattern
            pf = pt | (F.FSA_OUT_BF16 if self.out_bytes == 2 else 0)
            fwd.append((lib.fsa_forward_ex, (p["q"], p["k"], p["v"], dt, B, H, T, D, a,
                                             self.W, pf, p["out"], p["lse"], stream)))
            dq.append((lib.fsa_backward_dq_ex, (p["q"], p["k"], p["v"], p["dout"],
                                                p["lse"], dt, B, H, T, D, a, self.W, pt,
                                                p["dq"], p["ws"], nws, stream)))
            dkdv.append((lib.fsa_backward_dkdv_ex, (p["q"], p["k"], p["v"], p["dout"],
                                                    p["lse"], dt, B, H, T, D, a, self.W,
                                                    pt, p["dk"], p["dv"], p["dalpha"],
                                                    p["ws"], nws, stream)))
        # forward in layer order; backward in reverse layer order, dq stage then
        # dk/dv stage of each layer
        self.order = [("fwd",) + c for c in fwd]
        for l in reversed(range(len(self.L))):
            self.order += [("bwd_dq",) + dq[l], ("bwd_dkdv",) + dkdv[l]]

    def prepare_learned(self, torch, F, theta_map, optimizer, lr=1e-3):
        """Launches of a learned-alpha step on the same buffers: every layer's
        forward and backward read its tap table from device memory, and one
        fsa_theta_step updates every layer's theta from the layers' dalpha
        and writes the next step's alphas and tables. theta starts where
        alpha = 1."""
        import ctypes
        lib = F.lib()
        vp, f32 = ctypes.c_void_p, ctypes.c_float
        wl, L = self.wl, self.layers
        B, H, T, D = wl.B, wl.H, wl.T, wl.D
        dt = F.FSA_DTYPE_BF16 if wl.dtype == "bf16" else F.FSA_DTYPE_F32
        init = 1.0 if theta_map == F.FSA_THETA_CLAMP else 0.0
        self.theta = torch.full((L,), init, dtype=torch.float32, device="cuda")
        self.l_alpha = torch.empty(L, dtype=torch.float32, device="cuda")
        self.l_tables = torch.empty((L, F.FSA_TAP_TABLE_BYTES), dtype=torch.uint8, device="cuda")
        self.l_dalpha = torch.zeros(L, dtype=torch.float32, device="cuda")
        self.l_state = torch.zeros(F.theta_state_bytes(L), dtype=torch.uint8, device="cuda")
        F.fsa_theta_alpha(self.theta, theta_map, self.W, alpha=self.l_alpha, tables=self.l_tables)
        stream = vp(torch.cuda.current_stream().cuda_stream)
        fwd, bwd = [], []
        for l, t in enumerate(self.L):
            p = {n: vp(x.data_ptr()) for n, x in t.items()}
            tab = vp(self.l_tables[l].data_ptr())
            da = vp(self.l_dalpha[l:l + 1].data_ptr())
            fwd.append(("fwd", lib.fsa_forward_dev, (p["q"], p["k"], p["v"], dt, B, H, T, D,
                                                     tab, self.W, 0, p["out"], p["lse"],
                                                     stream)))
            bwd.append(("bwd", lib.fsa_backward_dev, (p["q"], p["k"], p["v"], p["dout"],
                                                      p["lse"], dt, B, H, T, D, tab, self.W,
                                                      p["dq"], p["dk"], p["dv"], da, p["ws"],
                                                      t["ws"].numel(), stream)))
        upd = ("theta_step", lib.fsa_theta_step,
               (vp(self.theta.data_ptr()), vp(self.l_dalpha.data_ptr()), L, theta_map,
                optimizer, f32(lr), f32(0.9), f32(0.999), f32(1e-8),
                vp(self.l_state.data_ptr()), self.W, F.FSA_PATTERN_FIB,
                vp(self.l_alpha.data_ptr()), vp(self.l_tables.data_ptr()), stream))
        self.order = fwd + bwd[::-1] + [upd]

    def step(self, ev=None):
        for name, fn, args in self.order:
            if ev is not None:
                ev.record(name)
            st = fn(*args)
            if st != 0:
                raise RuntimeError(f"{name} returned status {st}")
            if ev is not None:
                ev.record(Events.END)
        if ev is not None:
            ev.record(None)


class DecodeStack:
    """Device buffers of the decoding workload: one query per (b, h) and
    layer against the caches; DECODE_CACHES distinct layer caches serve the
    layers of one step in turn."""

    def __init__(self, wl, window, torch, F, I, pattern="fib"):
        import ctypes
        self.wl, self.W, self.layers = wl, window, wl.layers
        self.alphas = F.fsa_schedule(F.FSA_SCHEDULE_LINEAR, wl.layers)
        self.pattern = F.PATTERNS[pattern]
        B, H, T, D = wl.B, wl.H, wl.T, wl.D
        self.caches = []
        for c in range(I.DECODE_CACHES):
            x = I.decode_inputs(wl, c)
            t = {n: I.to_device(x[n], wl.dtype) for n in ("q", "k", "v")}
            t["pos"] = torch.from_numpy(x["pos"]).to("cuda")
            self.caches.append(t)
        self.positions = x["pos"]
        f32t = lambda *s: torch.empty(s, dtype=torch.float32, device="cuda")
        self.outs = [(f32t(B, H, D), f32t(B, H)) for _ in range(wl.layers)]
        lib = F.lib()
        vp, f32 = ctypes.c_void_p, ctypes.c_float
        dt = F.FSA_DTYPE_BF16 if wl.dtype == "bf16" else F.FSA_DTYPE_F32
        stream = vp(torch.cuda.current_stream().cuda_stream)
        self.order = []
        for l in range(wl.layers):
            t = self.caches[l % len(self.caches)]
            o, ls = self.outs[l]
            p = {n: vp(x.data_ptr()) for n, x in t.items()}
            self.order.append(("decode", lib.fsa_decode,
                               (p["q"], p["k"], p["v"], dt, B, H, T, D, p["pos"],
                                f32(float(self.alphas[l])), window, self.pattern,
                                vp(o.data_ptr()), vp(ls.data_ptr()), stream)))
        # rows each (b, h) query reads: its window rows and one or two rows per
        # reaching tap (two when the distance is fractional)
        self.rows_per_step = 0
        for l in range(wl.layers):
            c, tt, keep = F.fsa_offsets(float(self.alphas[l]), window, self.pattern)
            for i in self.positions:
                i = int(i)
                self.rows_per_step += H * (min(window, i + 1) + sum(
                    (2 if tt[n] != 0 else 1) for n in range(len(c))
                    if keep[n] and c[n] <= i))

    step = Stack.step

    def graph_ms(self, torch, reps):
        """Step time with the step's launches captured once in a HIP graph
        (torch.cuda.CUDAGraph) and replayed: the launches are re-marshalled
        onto the capture stream."""
        import ctypes
        s = torch.cuda.Stream()
        calls = [(fn, args[:-1] + (ctypes.c_void_p(s.cuda_stream),))
                 for _, fn, args in self.order]
        graph = torch.cuda.CUDAGraph()
        torch.cuda.synchronize()
        with torch.cuda.graph(graph, stream=s):
            for fn, a in calls:
                if fn(*a) != 0:
                    raise RuntimeError("launch failed during capture")
        for _ in range(3):
            graph.replay()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(reps):
            graph.replay()
        torch.cuda.synchronize()
        return (time.perf_counter() - t0) * 1e3 / reps

    def bytes_per_step(self):
        """Algorithmic bytes of one step: every row read once (K and V), the
        queries, out and lse."""
        wl = self.wl
        in_b = 2 if wl.dtype == "bf16" else 4
        per_query = wl.D * in_b + 4 * wl.D + 4
        return (self.rows_per_step * 2 * wl.D * in_b
                + wl.layers * wl.B * wl.H * per_query)


class RopeStack:
    """Device buffers of the RoPE pass over one workload's shape: per layer the
    pre-RoPE q and k (bf16, rotated into bf16 rows, "rope") and the fp32
    gradients dq and dk (turned back, "rope_inv"). `sets` distinct buffer
    sets (more than the Infinity Cache in all) serve the layers in turn."""

    def __init__(self, wl, torch, F, I, layers, sets):
        import ctypes
        self.wl, self.layers = wl, layers
        B, H, T, D = wl.B, wl.H, wl.T, wl.D
        self.sets = []
        # seeded N(0, 1) rows drawn on the device (the 65536-token size is too
        # large to draw on the host at bench start)
        gen = torch.Generator(device="cuda")
        gen.manual_seed(I.SEED_ROOT + wl.workload_id)
        for c in range(sets):
            draw = lambda dt: torch.randn((B, H, T, D), generator=gen, device="cuda").to(dt)
            t = {"q": draw(torch.bfloat16), "k": draw(torch.bfloat16),
                 "dq": draw(torch.float32), "dk": draw(torch.float32)}
            for n in ("q", "k"):
                t[n + "r"] = torch.empty_like(t[n])
            for n in ("dq", "dk"):
                t[n + "p"] = torch.empty_like(t[n])
            self.sets.append(t)
        lib = F.lib()
        vp, f32 = ctypes.c_void_p, ctypes.c_float
        stream = vp(torch.cuda.current_stream().cuda_stream)
        base = f32(wl.rope_base)
        bf, fp = F.FSA_DTYPE_BF16, F.FSA_DTYPE_F32
        self.order = []
        for l in range(layers):
            p = {n: vp(x.data_ptr()) for n, x in self.sets[l % sets].items()}
            for n in ("q", "k"):
                self.order.append(("rope", lib.fsa_rope, (p[n], bf, B, H, T, D, base, None,
                                                          0, p[n + "r"], bf, stream)))
        for l in reversed(range(layers)):
            p = {n: vp(x.data_ptr()) for n, x in self.sets[l % sets].items()}
            for n in ("dq", "dk"):
                self.order.append(("rope_inv", lib.fsa_rope, (p[n], fp, B, H, T, D, base,
                                                              None, 1, p[n + "p"], fp, stream)))

    step = Stack.step


class RopeLayerStack:
    """A layer with RoPE, forward and backward, both ways, on seeded N(0,1)
    rows drawn on the device before rotation:
      separate: the RoPE pass on q and k, forward, backward (dq and dk/dv
                stages), the inverse pass on dq and dk;
      fused:    the RoPE pass on k, the forward turning its query tiles (and
                writing the turned rows the backward reads), the backward
                turning dq and dk back at store time.
    `sets` buffer sets serve the layers in turn."""

    def __init__(self, wl, torch, F, I, layers, sets, fused, window=12):
        import ctypes
        self.wl, self.layers = wl, layers
        B, H, T, D = wl.B, wl.H, wl.T, wl.D
        gen = torch.Generator(device="cuda")
        gen.manual_seed(I.SEED_ROOT + 97 * wl.workload_id)
        bf, f32 = torch.bfloat16, torch.float32
        alphas = F.fsa_schedule(F.FSA_SCHEDULE_LINEAR, 16)
        nbytes = F.fsa_backward_workspace_size(B, H, T, D, F.FSA_DTYPE_BF16)
        self.sets = []
        for c in range(sets):
            draw = lambda: torch.randn((B, H, T, D), generator=gen, device="cuda").to(bf)
            t = {"qp": draw(), "kp": draw(), "v": draw(), "dout": draw()}
            for n in ("q", "k"):
                t[n] = torch.empty_like(t["qp"])
            for n in ("out", "dq", "dk", "dv", "dqp", "dkp"):
                t[n] = torch.empty((B, H, T, D), dtype=f32, device="cuda")
            t["lse"] = torch.empty((B, H, T), dtype=f32, device="cuda")
            t["da"] = torch.empty(1, dtype=f32, device="cuda")
            t["ws"] = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
            self.sets.append(t)
        lib = F.lib()
        vp, fl = ctypes.c_void_p, ctypes.c_float
        st = vp(torch.cuda.current_stream().cuda_stream)
        base = fl(wl.rope_base)
        dt = F.FSA_DTYPE_BF16
        self.order = []
        for l in range(layers):
            t = self.sets[l % sets]
            p = {n: vp(x.data_ptr()) for n, x in t.items()}
            a = fl(float(alphas[l % 16]))
            nws = t["ws"].numel()
            rope = lambda x, y, tin, inv: ("rope" if not inv else "rope_inv", lib.fsa_rope,
                                           (p[x], tin, B, H, T, D, base, None, inv, p[y], tin, st))
            if fused:
                self.order += [
                    rope("kp", "k", dt, 0),
                    ("fwd_rope", lib.fsa_forward_rope,
                     (p["qp"], p["k"], p["v"], dt, B, H, T, D, a, window, 0, base, None,
                      p["out"], p["lse"], p["q"], st)),
                    ("bwd_rope", lib.fsa_backward_rope,
                     (p["q"], p["k"], p["v"], p["dout"], p["lse"], dt, B, H, T, D, a, window,
                      0, base, None, p["dqp"], p["dkp"], p["dv"], p["da"], p["ws"], nws, st))]
            else:
                self.order += [
                    rope("qp", "q", dt, 0), rope("kp", "k", dt, 0),
                    ("fwd", lib.fsa_forward, (p["q"], p["k"], p["v"], dt, B, H, T, D, a, window,
                                              p["out"], p["lse"], st)),
                    ("bwd", lib.fsa_backward, (p["q"], p["k"], p["v"], p["dout"], p["lse"], dt,
                                               B, H, T, D, a, window, p["dq"], p["dk"],
                                               p["dv"], p["da"], p["ws"], nws, st)),
                    rope("dq", "dqp", F.FSA_DTYPE_F32, 1), rope("dk", "dkp", F.FSA_DTYPE_F32, 1)]

    step = Stack.step


class Events:
    """Timing events on the launch stream, created through HIP with
    hipEventDisableSystemFence (no cache writeback and invalidation at each
    record). Each launch is bracketed by an event before it and an event
    after it; the time between the two is that launch's time. Every record
    costs the command processor a few microseconds, and an event-to-event
    gap taken from one launch to the next would add that cost to every
    launch; with the pair it falls between launches instead. All events are
    created up front, so recording one costs the host only the enqueue."""

    DISABLE_SYSTEM_FENCE = 0x20000000
    END = ""                          # the event after a launch

    def __init__(self, torch, count):
        import ctypes
        self.ct = ctypes
        self.hip = ctypes.CDLL("libamdhip64.so")       # the runtime torch loaded
        self.stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
        self.pool = []
        for _ in range(count):
            e = ctypes.c_void_p()
            if self.hip.hipEventCreateWithFlags(ctypes.byref(e),
                                                ctypes.c_uint(self.DISABLE_SYSTEM_FENCE)) != 0:
                raise RuntimeError("hipEventCreateWithFlags failed")
            self.pool.append(e)
        self.marks = []

    def record(self, name):
        """An event before a launch (`name` = the launch's kernel), after it
        (END) or at the end of a step (None)."""
        e = self.pool[len(self.marks)]
        if self.hip.hipEventRecord(e, self.stream) != 0:
            raise RuntimeError("hipEventRecord failed")
        self.marks.append((name, e))

    def per_kernel_ms(self, skip_steps=1):
        """Median time of each kernel from the event before its launch to the
        event after it, over the recorded steps after the first `skip_steps`
        ones, and the launches counted. The median, not the mean: a host stall
        that drains the queue lands in whichever launch it falls in and would
        move a mean by its whole length."""
        gaps = {}
        f = self.ct.c_float()
        step = 0
        for (name, e0), (nxt, e1) in zip(self.marks, self.marks[1:]):
            if name is None:
                step += 1
                continue
            if name == self.END or nxt != self.END or step < skip_steps:
                continue
            if self.hip.hipEventElapsedTime(self.ct.byref(f), e0, e1) != 0:
                raise RuntimeError("hipEventElapsedTime failed")
            gaps.setdefault(name, []).append(f.value)
        med = {n: statistics.median(v) for n, v in gaps.items()}
        return med, {n: len(v) for n, v in gaps.items()}

    def close(self):
        for e in self.pool:
            self.hip.hipEventDestroy(e)
        self.pool = []


def time_stack(stack, steps, warmup, torch):
    """Step time on the host clock with no events between launches; then the
    per-kernel event medians over as many steps again (one more step is run
    first and dropped). Returns (ms per step, median ms per kernel, launches
    per step per kernel)."""
    for _ in range(warmup):
        stack.step()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        stack.step()
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    ms_step = (t1 - t0) * 1e3 / steps
    ev = Events(torch, (steps + 1) * (2 * len(stack.order) + 1))
    for _ in range(steps + 1):
        stack.step(ev)
    torch.cuda.synchronize()
    per_ms, counts = ev.per_kernel_ms(skip_steps=1)
    ev.close()
    per_step = {n: c // steps for n, c in counts.items()}
    return ms_step, per_ms, per_step


def consistency(ms_step, per_ms, per_step):
    """Self-check of the per-kernel figures: the kernel medians times their
    launches per step, summed, against the host-clock step time. The two
    measure the same launches; the kernel times leave out the short gaps
    between one launch's end and the next one's start, so the sum sits a few
    percent under the step time. A ratio outside 0.9-1.1 flags the line."""
    total = sum(per_ms[n] * per_step[n] for n in per_ms)
    ratio = total / ms_step if ms_step > 0 else float("nan")
    return {"sum_kernel_ms": round(total, 4), "ms_per_step": round(ms_step, 4),
            "ratio": round(ratio, 4), "ok": bool(0.9 <= ratio <= 1.1)}


def summarise(stack, ms_step, per_ms):
    wl = stack.wl
    th = wl.B * wl.H * wl.T                      # token-heads per layer call
    in_b = 2 if wl.dtype == "bf16" else 4
    sb = stage_bytes(wl.D, in_b, stack.out_bytes)
    ab = algo_bytes(wl.D, in_b, stack.out_bytes)
    kernels = {}
    for n, ms in per_ms.items():
        k = {"median_us": round(ms * 1e3, 3)}
        if n in sb:
            gbs = sb[n] * th / (ms * 1e-3) / 1e9
            k.update(bytes_per_launch=sb[n] * th, gbs=round(gbs, 1),
                     hbm_frac=round(gbs / HBM_PEAK_GBS, 4))
        kernels[n] = k
    fwd_ms = per_ms["fwd"]
    bwd_ms = per_ms["bwd_dq"] + per_ms["bwd_dkdv"]
    frac = {
        "fwd": round(ab["fwd"] * th / (fwd_ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
        "bwd": round(ab["bwd"] * th / (bwd_ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
        "fwd_bwd": round((ab["fwd"] + ab["bwd"]) * th / ((fwd_ms + bwd_ms) * 1e-3)
                         / 1e9 / HBM_PEAK_GBS, 4),
    }
    value = stack.layers * th / (ms_step * 1e-3)
    # the forward and the backward timed separately (event means per layer)
    passes = {"fwd": round(th / (fwd_ms * 1e-3), 1), "bwd": round(th / (bwd_ms * 1e-3), 1)}
    return value, kernels, frac, passes


def source_digest():
    h = hashlib.sha256()
    for p in KERNEL_SOURCES:
        if os.path.exists(p):
            h.update(open(p, "rb").read())
    return h.hexdigest()[:16]


def load_traffic(kernel, per_launch_tokens, workload):
    """HBM bytes per launch from the committed rocprofv3 counter summary of the
    kernel on `workload`, when it was taken on the current kernel source; else
    None. The summary holds one line per workload:
        hbm_bytes_per_token_head <workload>: <bytes>"""
    path = os.path.join(PROFILES, f"traffic_{kernel}.txt")
    if not os.path.exists(path):
        return None
    text = open(path).read()
    m = re.search(r"source_digest:\s*(\w+)", text)
    b = re.search(r"hbm_bytes_per_token_head\s+" + re.escape(workload)
                  + r":\s*([0-9.eE+-]+)", text)
    if not m or not b or m.group(1) != source_digest():
        return None
    return round(float(b.group(1)) * per_launch_tokens)


def copy_bandwidth(torch, nbytes=1 << 30, reps=10):
    """Achievable HBM bandwidth on this device for context: a plain 1 GiB
    device-to-device copy (read + write bytes over the mean copy time)."""
    src = torch.empty(nbytes, dtype=torch.uint8, device="cuda").fill_(1)
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        dst.copy_(src)
    e1.record()
    torch.cuda.synchronize()
    sec = e0.elapsed_time(e1) * 1e-3 / reps
    del src, dst
    torch.cuda.empty_cache()
    return round(2 * nbytes / sec / 1e9, 1)


# ------------------------------------------------------------- CPU baseline
TOL_MAX_ABS = {"bf16": 2e-3, "f32": 2e-5}
TOL_DALPHA_REL = 1e-3


def _oracle_layer(args):
    """The fp64 oracle's forward and backward over every (b, h) slab of one
    layer; when the GPU results of the layer are given, also their largest
    absolute difference from the oracle per output, and the oracle's dalpha
    (summed in a fixed order)."""
    import numpy as np
    from oracle import fsa_oracle as O
    q, k, v, g, alpha, W, base, mode, got = args
    B, H = q.shape[:2]
    errs = {n: 0.0 for n in ("out", "lse", "dq", "dk", "dv")}
    parts = []
    busy = 0.0
    for b in range(B):
        for h in range(H):
            t0 = time.perf_counter()
            sl = [x[b, h].astype(np.float64) for x in (q, k, v, g)]
            ro, rl = O.forward_slab(sl[0], sl[1], sl[2], alpha, W, base=base, mode=mode)
            rq, rk, rv, ra, _ = O.backward_slab(sl[0], sl[1], sl[2], sl[3], alpha, W,
                                                base=base, mode=mode)
            busy += time.perf_counter() - t0
            parts.append(ra)
            if got is not None:
                for n, r in (("out", ro), ("lse", rl), ("dq", rq), ("dk", rk), ("dv", rv)):
                    e = float(np.abs(got[n][b, h].astype(np.float64) - r).max())
                    errs[n] = max(errs[n], e)
    return busy, (errs if got is not None else None), math.fsum(parts)


def _noop(_):
    return os.getpid()


def cpu_baseline(stack, pattern="fib", passes=2, per_slab=False):
    """The fp64 oracle (forward + backward of every (b, h) slab) over every
    layer of the stack, `passes` times over the step, one layer per worker
    task (or one (b, h) slab per task with `per_slab`, for a single long
    layer); timed as a reported baseline. On its first pass the results of
    the layers whose GPU results the snapshot holds are compared with them
    (outside any timed GPU region). `stack` is a Stack.snapshot()."""
    wl, layers = stack.wl, stack.layers
    check_layers = tuple(stack.got)
    workers = max(1, min(16, len(os.sched_getaffinity(0))))
    for var in ("OMP_NUM_THREADS", "OPENBLAS_NUM_THREADS", "MKL_NUM_THREADS"):
        os.environ[var] = "1"
    base, _, mode = pattern.partition("-")
    mode = "round" if mode == "round" else "lerp"
    jobs, keys = [], []
    for p in range(passes):
        for l in range(layers):
            x = stack.host[l]
            got = stack.got[l] if (p == 0 and l in check_layers) else None
            slabs = ([(b, h) for b in range(wl.B) for h in range(wl.H)] if per_slab
                     else [None])
            for bh in slabs:
                cut = (lambda a: a) if bh is None else (
                    lambda a, b=bh[0], h=bh[1]: a[b:b + 1, h:h + 1])
                jobs.append((cut(x["q"]), cut(x["k"]), cut(x["v"]), cut(x["dout"]),
                             float(stack.alphas[l]), stack.W, base, mode,
                             None if got is None else {n: cut(a) for n, a in got.items()}))
                keys.append((p, l))
    ctx = multiprocessing.get_context("spawn")
    from concurrent.futures import ProcessPoolExecutor
    with ProcessPoolExecutor(max_workers=workers, mp_context=ctx) as ex:
        list(ex.map(_noop, range(workers * 2)))          # start every worker
        t0 = time.perf_counter()
        res = list(ex.map(_oracle_layer, jobs))
        wall = time.perf_counter() - t0
    th = passes * layers * wl.B * wl.H * wl.T
    unit = "(b,h) slab" if per_slab else "layer"
    base_line = {"value": round(th / wall, 1), "unit": "tokens·heads/s",
                 "cores": workers, "kind": "oracle",
                 "sample": (f"{passes} passes over {layers} layers x {wl.B * wl.H} (b,h) "
                            f"slabs of {wl.name} (W={stack.W}), forward+backward in "
                            f"fp64 numpy, one {unit} per task, {workers} spawned "
                            f"single-threaded workers; {wall:.1f} s wall, "
                            f"{sum(r[0] for r in res):.1f} s CPU")}
    parity = None
    if check_layers:
        errs = {n: 0.0 for n in ("out", "lse", "dq", "dk", "dv")}
        da_parts = {l: [] for l in check_layers}
        for (p, l), r in zip(keys, res):
            if p != 0 or l not in check_layers:
                continue
            for n in errs:
                errs[n] = max(errs[n], r[1][n])
            da_parts[l].append(r[2])
        da_rel = 0.0
        for l in check_layers:
            ref = math.fsum(da_parts[l])
            got_da = stack.da[l]
            if ref != 0.0:
                da_rel = max(da_rel, abs(got_da - ref) / abs(ref))
            elif got_da != 0.0:
                da_rel = float("inf")
        tol = TOL_MAX_ABS[wl.dtype]
        out_ok = stack.out_bytes == 4
        parity = {"layers": sorted(check_layers), "max_abs": {n: float(f"{e:.3g}") for n, e in errs.items()},
                  "dalpha_rel": float(f"{da_rel:.3g}"),
                  "tol": {"max_abs": tol, "dalpha_rel": TOL_DALPHA_REL},
                  "ok": bool(all(e <= tol for n, e in errs.items() if n != "out" or out_ok)
                             and da_rel <= TOL_DALPHA_REL)}
    return base_line, parity


# ------------------------------------------------------------- roofline
def roofline(stack, per_ms, kernels, traffic_ok):
    """Roofline object of the dominant kernel (the longest median launch):
    its algorithmic bytes per launch over that median, against the 8 TB/s HBM
    peak; traffic from the committed counter summary when it was taken on the
    current kernel source and workload, else null."""
    wl = stack.wl
    th = wl.B * wl.H * wl.T
    dom = max((n for n in per_ms if n in kernels and "gbs" in kernels[n]),
              key=lambda n: per_ms[n])
    achieved = kernels[dom]["gbs"]
    traffic = load_traffic(dom, th, wl.name) if traffic_ok else None
    return {"bound": "hbm", "kernel": dom, "achieved": achieved,
            "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": traffic,
            "algorithmic_bytes_per_launch": kernels[dom]["bytes_per_launch"],
            "median_launch_us": kernels[dom]["median_us"]}


def learned_leg(stack, res, args, wl, ms_step, torch, F):
    """The learned-alpha step (every layer's forward and backward reading its
    tap table from device memory, then one fsa_theta_step) on the static
    stack's buffers; the static launches are restored afterwards and one
    static step refreshes the results the oracle check reads."""
    stack.prepare_learned(torch, F, F.FSA_THETA_CLAMP, F.FSA_OPT_ADAM)

    ms_l, per_l, _ = time_stack(stack, args.steps, args.warmup, torch)
    alphas_now = stack.l_alpha.cpu().numpy()
    res["learned"] = {
        "workload": wl.name + " (learned alpha: clip map, Adam, theta from alpha = 1)",
        "ms_per_step": round(ms_l, 4), "static_ms_per_step": round(ms_step, 4),
        "ratio_to_static": round(ms_l / ms_step, 4),
        "value": round(args.layers * wl.B * wl.H * wl.T / (ms_l * 1e-3), 1),
        "median_us": {n: round(v * 1e3, 3) for n, v in per_l.items()},
        "alpha_range_after": [round(float(alphas_now.min()), 6), round(float(alphas_now.max()), 6)]}
    # back to the static schedule; one more static step refreshes the results
    # that the oracle check reads
    stack._prepare_calls(torch, F)
    stack.step()
    torch.cuda.synchronize()


# ------------------------------------------------------------- main
def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--layers", type=int, default=16)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--skip-t4096", action="store_true")
    ap.add_argument("--skip-decode", action="store_true")
    ap.add_argument("--skip-t65536", action="store_true")
    ap.add_argument("--skip-rope", action="store_true")
    ap.add_argument("--skip-learned", action="store_true",
                    help="leave out the learned-alpha step")
    ap.add_argument("--skip-sweep", action="store_true",
                    help="leave out the T4096 window sweep (other tap counts on the "
                         "same grid, which counter runs would mix in)")
    ap.add_argument("--out-bf16", action="store_true",
                    help="the forward writes out in bf16 (FSA_OUT_BF16)")
    ap.add_argument("--pattern", default="fib",
                    choices=["fib", "fib-round", "pow2", "pow2-round"],
                    help="tap pattern: Fibonacci or power-of-two base, "
                         "interpolated or rounded offsets (default fib)")
    ap.add_argument("--skip-c1", action="store_true",
                    help="leave out the fp32 B1 H4 T256 layer (alpha = 1, W = 8)")
    ap.add_argument("--seed", type=int, default=None,
                    help="seed root of the synthetic inputs (default: the recipe's)")
    ap.add_argument("--jsonl", default=None,
                    help="also write one JSON record per workload to this file")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="also run a plain 1 GiB device copy (3 launches), whose "
                         "FETCH_SIZE/WRITE_SIZE counters scale the kernels' counters "
                         "to bytes in a rocprofv3 --pmc run")
    args = ap.parse_args()
    if args.gpus != 1:
        print("bench.py measures one GPU: this library has no multi-GPU path "
              "(the heads shard with no exchange; see the design notes). "
              "Run with --gpus 1.", file=sys.stderr)
        sys.exit(2)

    import torch

    from static_pattern_sparse_amd import fsa as F
    from static_pattern_sparse_amd import inputs as I
    torch.cuda.set_device(0)
    F.lib()
    if args.calibrate_copy:
        src = torch.empty(1 << 30, dtype=torch.uint8, device="cuda").fill_(1)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
        torch.cuda.empty_cache()

    wl = I.WORKLOADS["linear16_bwd_bf16_b8h8t1024d64_w12"]
    stack = Stack(wl, 12, args.layers, torch, F, I, args.pattern, args.out_bf16, args.seed)
    print(f"[bench] {wl.name}: {args.layers} layers resident", file=sys.stderr, flush=True)
    ms_step, per_ms, counts = time_stack(stack, args.steps, args.warmup, torch)
    value, kernels, frac, passes = summarise(stack, ms_step, per_ms)
    print(f"[bench] {ms_step:.3f} ms/step", file=sys.stderr, flush=True)

    # the committed counter summaries were taken with the Fibonacci table
    traffic_ok = args.pattern == "fib" and not args.out_bf16
    roof = roofline(stack, per_ms, kernels, traffic_ok)

    res = {
        "metric": METRIC, "value": round(value, 1), "unit": "tokens·heads/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic (seeded N(0,1) post-RoPE q, k; v; dout)",
        "config": {"workload": wl.name, "B": wl.B, "H": wl.H, "T": wl.T, "D": wl.D,
                   "W": 12, "layers": args.layers, "schedule": wl.schedule,
                   "pattern": args.pattern,
                   "out_dtype": "bf16" if args.out_bf16 else "f32",
                   "pass": "forward+backward"},
        "roofline": roof,
        "consistency": consistency(ms_step, per_ms, counts),
        "hbm_frac": frac,
        "pass_tokens_heads_per_s": passes,
        # context: a plain 1 GiB device copy on the same GPU (read + write)
        "copy_gbs": copy_bandwidth(torch),
        "kernels": kernels,
        "launches_per_step": counts,
    }
    # the learned-alpha step on the same buffers (Adam on theta with the clip
    # map): the layers' tables on the device, one update launch per step
    if not args.skip_learned:
        learned_leg(stack, res, args, wl, ms_step, torch, F)
    # the first and the last layer's GPU results, for the oracle check that
    # runs with the CPU baseline after every GPU leg
    snap1024 = stack.snapshot((0, args.layers - 1)) if not args.no_cpu_baseline else None
    del stack
    torch.cuda.empty_cache()

    if not args.skip_t4096:
        wl2 = I.WORKLOADS["coprime16_bf16_b4h8t4096d64_w6-12"]
        st2 = Stack(wl2, 12, args.layers, torch, F, I, args.pattern, args.out_bf16, args.seed)
        print(f"[bench] {wl2.name} W=12 resident", file=sys.stderr, flush=True)
        ms2, per2, cnt2 = time_stack(st2, max(1, args.steps // 2), max(1, args.warmup), torch)
        v2, k2, f2, p2 = summarise(st2, ms2, per2)
        res["t4096"] = {"workload": wl2.name + " (W=12)", "value": round(v2, 1),
                        "ms_per_step": round(ms2, 4),
                        "roofline": roofline(st2, per2, k2, traffic_ok),
                        "consistency": consistency(ms2, per2, cnt2),
                        "hbm_frac": f2,
                        "pass_tokens_heads_per_s": p2, "kernels": k2}
        snap4096 = (st2.snapshot((1, args.layers - 1))
                    if not args.no_cpu_baseline else None)
        # the window sweep of the same stack: forward launches only (the
        # inputs do not depend on W), host clock over back-to-back launches
        sweep = {}
        for W in (() if args.skip_sweep else (6, 8, 10, 12)):
            st2.W = W
            st2._prepare_calls(torch, F)
            fwd = [(fn, a) for name, fn, a in st2.order if name == "fwd"]
            for fn, a in fwd:
                fn(*a)
            torch.cuda.synchronize()
            reps = max(2, args.steps // 2)
            t0 = time.perf_counter()
            for _ in range(reps):
                for fn, a in fwd:
                    fn(*a)
            torch.cuda.synchronize()
            us = (time.perf_counter() - t0) * 1e6 / (reps * len(fwd))
            ab = algo_bytes(wl2.D, 2, st2.out_bytes)["fwd"] * wl2.B * wl2.H * wl2.T
            sweep[f"W{W}"] = {"fwd_us": round(us, 2),
                              "hbm_frac": round(ab / (us * 1e-6) / 1e9 / HBM_PEAK_GBS, 4)}
        if sweep:
            res["t4096"]["window_sweep_forward"] = sweep
        del st2
        torch.cuda.empty_cache()

    if not args.skip_t65536:
        wl4 = I.WORKLOADS["linear16_bf16_b1h16t65536d128_w12"]
        st4 = Stack(wl4, 12, 1, torch, F, I, args.pattern, args.out_bf16, args.seed)
        print(f"[bench] {wl4.name} (one layer) resident", file=sys.stderr, flush=True)
        ms4, per4, cnt4 = time_stack(st4, max(2, args.steps // 2), 1, torch)
        v4, k4, f4, p4 = summarise(st4, ms4, per4)
        res["t65536"] = {"workload": wl4.name + " (one layer, alpha of layer 0)",
                         "value": round(v4, 1), "ms_per_step": round(ms4, 4),
                         "consistency": consistency(ms4, per4, cnt4),
                         "hbm_frac": f4, "pass_tokens_heads_per_s": p4, "kernels": k4}
        # every head of the layer, for the oracle check after the GPU legs
        snap65536 = st4.snapshot((0,)) if not args.no_cpu_baseline else None
        del st4
        torch.cuda.empty_cache()

    if not args.skip_c1:
        # the fp32 layer: alpha = 1, integer offsets, the row-group kernels
        wl1 = I.WORKLOADS["fixed_f32_b1h4t256d64_w8"]
        st1 = Stack(wl1, 8, 1, torch, F, I, args.pattern, False, args.seed)
        print(f"[bench] {wl1.name} resident", file=sys.stderr, flush=True)
        ms1, per1, cnt1 = time_stack(st1, max(20, args.steps * 5), max(5, args.warmup), torch)
        v1, k1, f1, p1 = summarise(st1, ms1, per1)
        res["c1"] = {"workload": wl1.name + " (one layer, alpha = 1, W = 8, fp32)",
                     "value": round(v1, 1), "ms_per_step": round(ms1, 4),
                     "consistency": consistency(ms1, per1, cnt1), "hbm_frac": f1,
                     "pass_tokens_heads_per_s": p1, "kernels": k1}
        snap_c1 = st1.snapshot((0,)) if not args.no_cpu_baseline else None
        del st1
        torch.cuda.empty_cache()

    if not args.skip_decode:
        wl3 = I.WORKLOADS["decode16_bf16_b8h8t4096d64_w12"]
        st3 = DecodeStack(wl3, 12, torch, F, I, args.pattern)
        print(f"[bench] {wl3.name} resident", file=sys.stderr, flush=True)
        ms3, per3, _ = time_stack(st3, max(20, args.steps * 5), max(5, args.warmup), torch)
        launch_us = per3["decode"] * 1e3
        nbytes = st3.bytes_per_step() / wl3.layers
        graph_ms = st3.graph_ms(torch, max(20, args.steps * 5))
        res["decode"] = {
            "workload": wl3.name, "layers": wl3.layers,
            "positions": [int(p) for p in st3.positions],
            "us_per_step": round(ms3 * 1e3, 2),
            "tokens_per_s": round(wl3.B / (ms3 * 1e-3), 1),
            "graph_us_per_step": round(graph_ms * 1e3, 2),
            "median_launch_us": round(launch_us, 3),
            "algorithmic_bytes_per_launch": int(nbytes),
            "gbs": round(nbytes / (launch_us * 1e-6) / 1e9, 1),
            "bound": "latency"}
        del st3
        torch.cuda.empty_cache()

    if not args.skip_rope:
        res["rope"] = {}
        wl5 = I.WORKLOADS["linear16_bf16_b1h16t65536d128_w12"]
        for key, w, layers, sets in (("t1024", wl, wl.layers, 4), ("t65536", wl5, 2, 2)):
            st5 = RopeStack(w, torch, F, I, layers, sets)
            print(f"[bench] rope pass {key} resident", file=sys.stderr, flush=True)
            ms5, per5, _ = time_stack(st5, max(4, args.steps), max(2, args.warmup), torch)
            elems = w.B * w.H * w.T * w.D
            rope = {"workload": f"rope_b{w.B}h{w.H}t{w.T}d{w.D}_base{int(w.rope_base)}",
                    "launches_per_step": len(st5.order), "ms_per_step": round(ms5, 4)}
            for name, nbytes in (("rope", elems * (2 + 2)), ("rope_inv", elems * (4 + 4))):
                us = per5[name] * 1e3
                gbs = nbytes / (us * 1e-6) / 1e9
                rope[name] = {"median_launch_us": round(us, 3),
                              "algorithmic_bytes_per_launch": nbytes,
                              "gbs": round(gbs, 1), "hbm_frac": round(gbs / HBM_PEAK_GBS, 4)}
            res["rope"][key] = rope
            del st5
            torch.cuda.empty_cache()
            # a layer with RoPE both ways: the separate passes, or the rotation
            # fused where the rows sit in registers (only the key rows keep a pass)
            both = {}
            for fused in (False, True):
                st6 = RopeLayerStack(w, torch, F, I, layers, sets, fused)
                ms6, per6, _ = time_stack(st6, max(4, args.steps), max(2, args.warmup), torch)
                both["fused" if fused else "separate"] = {
                    "ms_per_layer": round(ms6 / layers, 4),
                    "median_us": {n: round(v * 1e3, 3) for n, v in per6.items()}}
                del st6
                torch.cuda.empty_cache()
            both["fused_over_separate"] = round(both["fused"]["ms_per_layer"]
                                                / both["separate"]["ms_per_layer"], 4)
            res["rope"][key]["layer_fwd_bwd"] = both

    if not args.no_cpu_baseline:
        print("[bench] cpu baseline and oracle check", file=sys.stderr, flush=True)
        res["cpu_baseline"], res["parity"] = cpu_baseline(snap1024, args.pattern, passes=2)
        if not args.skip_t4096:
            cb, par = cpu_baseline(snap4096, args.pattern, passes=1)
            res["t4096"]["cpu_baseline"] = cb
            res["t4096"]["parity"] = par
        if not args.skip_t65536:
            cb, par = cpu_baseline(snap65536, args.pattern, passes=1, per_slab=True)
            res["t65536"]["cpu_baseline"] = cb
            res["t65536"]["parity"] = par
        if not args.skip_c1:
            cb, par = cpu_baseline(snap_c1, args.pattern, passes=20)
            res["c1"]["cpu_baseline"] = cb
            res["c1"]["parity"] = par
    else:
        res["cpu_baseline"] = None
    res["seed_root"] = I.SEED_ROOT if args.seed is None else args.seed
    if args.jsonl:
        write_jsonl(args.jsonl, res)
    print(json.dumps(res), flush=True)


def write_jsonl(path, res):
    """One record per workload of the run (the configurations and the other
    legs), each with the run's seed root, appended to `path`."""
    main_keys = ("workload", "value", "ms_per_step", "roofline", "consistency",
                 "hbm_frac", "pass_tokens_heads_per_s", "kernels", "parity",
                 "cpu_baseline")
    head = {k: res[k] for k in main_keys if k in res}
    head["workload"] = res["config"]["workload"]
    records = [("C2+C4 forward+backward", head)]
    for key, label in (("c1", "C1"), ("t4096", "C3 forward+backward"),
                       ("t65536", "C5 forward+backward, one layer"), ("decode", "decoding step"),
                       ("learned", "learned alpha step"), ("rope", "RoPE")):
        if key in res:
            records.append((label, res[key]))
    with open(path, "a") as fh:
        for label, rec in records:
            fh.write(json.dumps({"record": label, "seed_root": res["seed_root"], **rec}) + "\n")


if __name__ == "__main__":
    main()
