"""Thin Python binding of libfsa's C ABI (argument marshalling only).

The names mirror the C entry points declared in include/fsa.h. Tensors are
torch tensors on the GPU; torch supplies device memory and the current stream,
and every step of the computation runs in libfsa's HIP kernels. There is no
fallback: if libfsa.so is missing or fails to load, every call raises.
"""

from __future__ import annotations

import ctypes
import os

import numpy as np

FSA_OK = 0
FSA_ERR_INVALID_ARG = 1
FSA_ERR_UNSUPPORTED = 2
FSA_ERR_WORKSPACE = 3
FSA_ERR_HIP = 4
FSA_ERR_SCRATCH = 5
FSA_NOALLOC_SCRATCH_BYTES = 16 << 20

FSA_SCHEDULE_FIXED = 0
FSA_SCHEDULE_LINEAR = 1
FSA_SCHEDULE_COPRIME = 2

FSA_DTYPE_F32 = 0
FSA_DTYPE_BF16 = 1

NUM_TAPS = 15

# tap patterns (base | mode), as in include/fsa.h
FSA_BASE_FIBONACCI = 0
FSA_BASE_POW2 = 1
FSA_MODE_LERP = 0
FSA_MODE_ROUND = 2
FSA_PATTERN_FIB = FSA_BASE_FIBONACCI | FSA_MODE_LERP
FSA_OUT_BF16 = 4
# learned alpha: theta -> alpha maps, optimizers, device record sizes
FSA_THETA_CLAMP = 0
FSA_THETA_TANH = 1
FSA_OPT_SGD = 0
FSA_OPT_ADAM = 1
FSA_TAP_TABLE_BYTES = 256


def theta_state_bytes(num_layers):
    """FSA_THETA_STATE_BYTES(L): m[L], v[L] and the update count."""
    return 8 * int(num_layers) + 16


PATTERNS = {"fib": FSA_PATTERN_FIB,
            "fib-round": FSA_BASE_FIBONACCI | FSA_MODE_ROUND,
            "pow2": FSA_BASE_POW2 | FSA_MODE_LERP,
            "pow2-round": FSA_BASE_POW2 | FSA_MODE_ROUND}

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libfsa.so")
EXPORTS = ("fsa_schedule", "fsa_offsets", "fsa_offsets_ex", "fsa_forward",
           "fsa_forward_ex", "fsa_backward_workspace_size", "fsa_backward",
           "fsa_backward_ex", "fsa_backward_dq", "fsa_backward_dq_ex",
           "fsa_backward_dkdv", "fsa_backward_dkdv_ex", "fsa_backward_noalloc",
           "fsa_decode", "fsa_theta_alpha", "fsa_theta_step", "fsa_forward_dev",
           "fsa_backward_dev", "fsa_forward_rope", "fsa_backward_rope",
           "fsa_rope", "fsa_status_string", "fsa_last_hip_error")

_lib = None


class FsaError(RuntimeError):
    def __init__(self, fn, status, lib):
        msg = lib.fsa_status_string(status).decode()
        if status == FSA_ERR_HIP:
            msg += f" (hip error {lib.fsa_last_hip_error()})"
        super().__init__(f"{fn}: {msg}")
        self.status = status


def lib():
    """Open libfsa.so once and declare the C signatures."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                           "`python -m static_pattern_sparse_amd.build_lib`")
    # torch first: its HIP runtime is then the one libfsa binds to (same
    # soname). Loaded the other way round, the process would hold two HIP
    # runtimes, and torch's streams and memory would be foreign to libfsa's.
    import torch  # noqa: F401
    L = ctypes.CDLL(LIB_PATH)
    vp, i32, f32 = ctypes.c_void_p, ctypes.c_int, ctypes.c_float
    L.fsa_schedule.argtypes = [i32, i32, f32, f32, i32, ctypes.POINTER(f32)]
    L.fsa_schedule.restype = i32
    L.fsa_offsets.argtypes = [f32, i32, ctypes.POINTER(ctypes.c_int32),
                              ctypes.POINTER(f32), ctypes.POINTER(ctypes.c_uint8)]
    L.fsa_offsets.restype = i32
    L.fsa_offsets_ex.argtypes = [i32] + L.fsa_offsets.argtypes
    L.fsa_offsets_ex.restype = i32
    L.fsa_forward.argtypes = [vp, vp, vp, i32, i32, i32, i32, i32, f32, i32,
                              vp, vp, vp]
    L.fsa_forward.restype = i32
    L.fsa_backward_workspace_size.argtypes = [i32, i32, i32, i32, i32]
    L.fsa_backward_workspace_size.restype = ctypes.c_size_t
    L.fsa_backward.argtypes = [vp, vp, vp, vp, vp, i32, i32, i32, i32, i32,
                               f32, i32, vp, vp, vp, vp, vp, ctypes.c_size_t, vp]
    L.fsa_backward.restype = i32
    L.fsa_backward_dq.argtypes = [vp, vp, vp, vp, vp, i32, i32, i32, i32, i32,
                                  f32, i32, vp, vp, ctypes.c_size_t, vp]
    L.fsa_backward_dq.restype = i32
    L.fsa_backward_dkdv.argtypes = [vp, vp, vp, vp, vp, i32, i32, i32, i32, i32,
                                    f32, i32, vp, vp, vp, vp, ctypes.c_size_t, vp]
    L.fsa_backward_dkdv.restype = i32
    # _ex variants: the tap pattern follows `window` (argument 10 or 12)
    L.fsa_forward_ex.argtypes = L.fsa_forward.argtypes[:10] + [i32] + L.fsa_forward.argtypes[10:]
    L.fsa_forward_ex.restype = i32
    for name in ("fsa_backward", "fsa_backward_dq", "fsa_backward_dkdv"):
        base = getattr(L, name).argtypes
        ex = getattr(L, name + "_ex")
        ex.argtypes = base[:12] + [i32] + base[12:]
        ex.restype = i32
    L.fsa_backward_noalloc.argtypes = [vp, vp, vp, vp, vp, i32, i32, i32, i32, i32,
                                       f32, i32, i32, vp, vp, vp, vp, vp]
    L.fsa_backward_noalloc.restype = i32
    L.fsa_theta_alpha.argtypes = [vp, i32, i32, i32, i32, vp, vp, vp]
    L.fsa_theta_alpha.restype = i32
    L.fsa_theta_step.argtypes = [vp, vp, i32, i32, i32, f32, f32, f32, f32, vp, i32,
                                 i32, vp, vp, vp]
    L.fsa_theta_step.restype = i32
    L.fsa_forward_dev.argtypes = [vp, vp, vp, i32, i32, i32, i32, i32, vp, i32, i32,
                                  vp, vp, vp]
    L.fsa_forward_dev.restype = i32
    L.fsa_backward_dev.argtypes = [vp, vp, vp, vp, vp, i32, i32, i32, i32, i32, vp,
                                   i32, vp, vp, vp, vp, vp, ctypes.c_size_t, vp]
    L.fsa_backward_dev.restype = i32
    L.fsa_forward_rope.argtypes = [vp, vp, vp, i32, i32, i32, i32, i32, f32, i32, i32,
                                   f32, vp, vp, vp, vp, vp]
    L.fsa_forward_rope.restype = i32
    L.fsa_backward_rope.argtypes = [vp, vp, vp, vp, vp, i32, i32, i32, i32, i32, f32,
                                    i32, i32, f32, vp, vp, vp, vp, vp, vp,
                                    ctypes.c_size_t, vp]
    L.fsa_backward_rope.restype = i32
    L.fsa_decode.argtypes = [vp, vp, vp, i32, i32, i32, i32, i32, vp, f32, i32,
                             i32, vp, vp, vp]
    L.fsa_decode.restype = i32
    L.fsa_rope.argtypes = [vp, i32, i32, i32, i32, i32, f32, vp, i32, vp, i32, vp]
    L.fsa_rope.restype = i32
    L.fsa_status_string.argtypes = [i32]
    L.fsa_status_string.restype = ctypes.c_char_p
    L.fsa_last_hip_error.argtypes = []
    L.fsa_last_hip_error.restype = i32
    _lib = L
    return L


def _check(fn, status):
    if status != FSA_OK:
        raise FsaError(fn, status, lib())


def fsa_schedule(kind, num_layers=16, alpha_min=0.5, alpha_max=1.5, stride=7):
    out = np.zeros(num_layers, dtype=np.float32)
    st = lib().fsa_schedule(int(kind), int(num_layers), float(alpha_min),
                            float(alpha_max), int(stride),
                            out.ctypes.data_as(ctypes.POINTER(ctypes.c_float)))
    _check("fsa_schedule", st)
    return out


def fsa_offsets(alpha, window, pattern=FSA_PATTERN_FIB):
    c = np.zeros(NUM_TAPS, dtype=np.int32)
    t = np.zeros(NUM_TAPS, dtype=np.float32)
    keep = np.zeros(NUM_TAPS, dtype=np.uint8)
    st = lib().fsa_offsets_ex(int(pattern), float(alpha), int(window),
                           c.ctypes.data_as(ctypes.POINTER(ctypes.c_int32)),
                           t.ctypes.data_as(ctypes.POINTER(ctypes.c_float)),
                           keep.ctypes.data_as(ctypes.POINTER(ctypes.c_uint8)))
    _check("fsa_offsets", st)
    return c, t, keep.astype(bool)


def _dtype_code(t):
    import torch
    if t.dtype == torch.float32:
        return FSA_DTYPE_F32
    if t.dtype == torch.bfloat16:
        return FSA_DTYPE_BF16
    raise TypeError(f"unsupported dtype {t.dtype}")


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    import torch
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def _shape(q):
    if q.dim() != 4:
        raise ValueError("expected [B, H, T, D] tensors")
    for x in (q,):
        if not x.is_cuda or not x.is_contiguous():
            raise ValueError("tensors must be contiguous CUDA/HIP tensors")
    return tuple(int(s) for s in q.shape)


def _need(t, shape, dtype, name):
    """A caller-supplied device tensor must have exactly the shape and dtype
    the C ABI assumes for that pointer (the library sees only addresses)."""
    import torch
    if not isinstance(t, torch.Tensor) or not t.is_cuda or not t.is_contiguous():
        raise ValueError(f"{name} must be a contiguous device tensor")
    if tuple(t.shape) != tuple(shape) or t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype} of shape {tuple(shape)}, "
                         f"got {t.dtype} {tuple(t.shape)}")
    return t


def _rows(q, others):
    for x in others:
        if x.shape != q.shape or x.dtype != q.dtype or not x.is_contiguous() or not x.is_cuda:
            raise ValueError("q, k, v (and dout) must share shape and dtype and be "
                             "contiguous device tensors")


def _workspace(ws, nbytes):
    if not ws.is_cuda or not ws.is_contiguous():
        raise ValueError("workspace must be a contiguous device tensor")
    if ws.numel() * ws.element_size() < nbytes:
        raise ValueError(f"workspace needs {nbytes} bytes")
    return ws


def _out_buffer(out, out_dtype, shape, device, pattern):
    """The output tensor (fp32 or bf16) and the flags that describe it."""
    import torch
    if out is None:
        dt = torch.float32 if out_dtype is None else out_dtype
        out = torch.empty(shape, dtype=dt, device=device)
    if out.dtype not in (torch.float32, torch.bfloat16):
        raise TypeError("out must be float32 or bfloat16")
    if tuple(out.shape) != tuple(shape) or not out.is_contiguous():
        raise ValueError(f"out must be a contiguous {tuple(shape)} tensor")
    flags = int(pattern) & ~FSA_OUT_BF16
    if out.dtype == torch.bfloat16:
        flags |= FSA_OUT_BF16
    return out, flags


def fsa_forward(q, k, v, alpha, window, out=None, lse=None, stream=None,
                pattern=FSA_PATTERN_FIB, out_dtype=None):
    """out [B,H,T,D] (fp32, or bf16 with out_dtype=torch.bfloat16 or a bf16
    `out`) and lse [B,H,T] fp32 of one layer."""
    import torch
    B, H, T, D = _shape(q)
    _rows(q, (k, v))
    out, flags = _out_buffer(out, out_dtype, (B, H, T, D), q.device, pattern)
    if lse is None:
        lse = torch.empty((B, H, T), dtype=torch.float32, device=q.device)
    _need(lse, (B, H, T), torch.float32, "lse")
    st = lib().fsa_forward_ex(_ptr(q), _ptr(k), _ptr(v), _dtype_code(q), B, H,
                              T, D, float(alpha), int(window), flags,
                              _ptr(out), _ptr(lse), _stream(stream))
    _check("fsa_forward", st)
    return out, lse


def fsa_backward_workspace_size(B, H, T, D, dtype_code):
    return int(lib().fsa_backward_workspace_size(int(B), int(H), int(T), int(D),
                                                 int(dtype_code)))


def fsa_backward(q, k, v, dout, lse, alpha, window, dq=None, dk=None, dv=None,
                 dalpha=None, workspace=None, stream=None,
                 pattern=FSA_PATTERN_FIB):
    """dq, dk, dv [B,H,T,D] fp32 and dalpha [1] fp32 of one layer."""
    import torch
    B, H, T, D = _shape(q)
    _rows(q, (k, v, dout))
    dt = _dtype_code(q)
    f32 = torch.float32
    mk = lambda: torch.empty((B, H, T, D), dtype=f32, device=q.device)
    dq = mk() if dq is None else _need(dq, (B, H, T, D), f32, "dq")
    dk = mk() if dk is None else _need(dk, (B, H, T, D), f32, "dk")
    dv = mk() if dv is None else _need(dv, (B, H, T, D), f32, "dv")
    _need(lse, (B, H, T), f32, "lse")
    if dalpha is None:
        dalpha = torch.empty(1, dtype=f32, device=q.device)
    _need(dalpha, (1,), f32, "dalpha")
    nbytes = fsa_backward_workspace_size(B, H, T, D, dt)
    if workspace is None:
        workspace = torch.empty(max(nbytes, 1), dtype=torch.uint8, device=q.device)
    _workspace(workspace, nbytes)
    st = lib().fsa_backward_ex(_ptr(q), _ptr(k), _ptr(v), _ptr(dout), _ptr(lse),
                            dt, B, H, T, D, float(alpha), int(window),
                            int(pattern), _ptr(dq),
                            _ptr(dk), _ptr(dv), _ptr(dalpha), _ptr(workspace),
                            workspace.numel() * workspace.element_size(),
                            _stream(stream))
    _check("fsa_backward", st)
    return dq, dk, dv, dalpha


def fsa_backward_noalloc(q, k, v, dout, lse, alpha, window, dq, dk, dv, dalpha,
                         stream=None, pattern=FSA_PATTERN_FIB):
    """fsa_backward without a workspace: the library's fixed device scratch
    serves instead, and nothing is allocated (dq, dk, dv [B,H,T,D] fp32 and
    dalpha [1] fp32 are caller-supplied). Calls that overlap on one GPU race."""
    import torch
    B, H, T, D = _shape(q)
    _rows(q, (k, v, dout))
    f32 = torch.float32
    _need(dq, (B, H, T, D), f32, "dq")
    _need(dk, (B, H, T, D), f32, "dk")
    _need(dv, (B, H, T, D), f32, "dv")
    _need(lse, (B, H, T), f32, "lse")
    _need(dalpha, (1,), f32, "dalpha")
    st = lib().fsa_backward_noalloc(_ptr(q), _ptr(k), _ptr(v), _ptr(dout), _ptr(lse),
                                    _dtype_code(q), B, H, T, D, float(alpha),
                                    int(window), int(pattern), _ptr(dq), _ptr(dk),
                                    _ptr(dv), _ptr(dalpha), _stream(stream))
    _check("fsa_backward_noalloc", st)
    return dq, dk, dv, dalpha


def _ws_bytes(ws):
    return ws.numel() * ws.element_size()


def fsa_backward_dq(q, k, v, dout, lse, alpha, window, dq, workspace,
                    stream=None, pattern=FSA_PATTERN_FIB):
    """Stage 1 of the backward pass: dq, plus per-row terms and dalpha
    partials in `workspace`."""
    import torch
    B, H, T, D = _shape(q)
    _rows(q, (k, v, dout))
    _need(lse, (B, H, T), torch.float32, "lse")
    _need(dq, (B, H, T, D), torch.float32, "dq")
    _workspace(workspace, fsa_backward_workspace_size(B, H, T, D, _dtype_code(q)))
    st = lib().fsa_backward_dq_ex(_ptr(q), _ptr(k), _ptr(v), _ptr(dout),
                               _ptr(lse), _dtype_code(q), B, H, T, D,
                               float(alpha), int(window), int(pattern),
                               _ptr(dq), _ptr(workspace),
                               _ws_bytes(workspace), _stream(stream))
    _check("fsa_backward_dq", st)


def fsa_backward_dkdv(q, k, v, dout, lse, alpha, window, dk, dv, dalpha,
                      workspace, stream=None, pattern=FSA_PATTERN_FIB):
    """Stage 2 of the backward pass: dk, dv, and dalpha[0] from the stage-1
    partials."""
    import torch
    B, H, T, D = _shape(q)
    _rows(q, (k, v, dout))
    _need(lse, (B, H, T), torch.float32, "lse")
    _need(dk, (B, H, T, D), torch.float32, "dk")
    _need(dv, (B, H, T, D), torch.float32, "dv")
    _need(dalpha, (1,), torch.float32, "dalpha")
    _workspace(workspace, fsa_backward_workspace_size(B, H, T, D, _dtype_code(q)))
    st = lib().fsa_backward_dkdv_ex(_ptr(q), _ptr(k), _ptr(v), _ptr(dout),
                                 _ptr(lse), _dtype_code(q), B, H, T, D,
                                 float(alpha), int(window), int(pattern),
                                 _ptr(dk), _ptr(dv),
                                 _ptr(dalpha), _ptr(workspace),
                                 _ws_bytes(workspace), _stream(stream))
    _check("fsa_backward_dkdv", st)


def fsa_decode(q, k_cache, v_cache, pos, alpha, window, out=None, lse=None,
               stream=None, pattern=FSA_PATTERN_FIB, out_dtype=None):
    """One decoding step: out [B,H,D] fp32 and lse [B,H] fp32 of the queries
    q [B,H,D] at positions pos (int32 [B] on the device) against the caches
    [B,H,T_cap,D]."""
    import torch
    if q.dim() != 3 or k_cache.dim() != 4:
        raise ValueError("expected q [B, H, D] and caches [B, H, T_cap, D]")
    B, H, T_cap, D = (int(s) for s in k_cache.shape)
    if tuple(q.shape) != (B, H, D) or v_cache.shape != k_cache.shape:
        raise ValueError("q, k_cache, v_cache shapes disagree")
    for x in (q, k_cache, v_cache):
        if not x.is_cuda or not x.is_contiguous() or x.dtype != q.dtype:
            raise ValueError("q and the caches must be contiguous device tensors of one dtype")
    if pos.dtype != torch.int32 or tuple(pos.shape) != (B,) or not pos.is_cuda:
        raise ValueError("pos must be an int32 device tensor of shape [B]")
    out, flags = _out_buffer(out, out_dtype, (B, H, D), q.device, pattern)
    if lse is None:
        lse = torch.empty((B, H), dtype=torch.float32, device=q.device)
    _need(lse, (B, H), torch.float32, "lse")
    st = lib().fsa_decode(_ptr(q), _ptr(k_cache), _ptr(v_cache), _dtype_code(q),
                          B, H, T_cap, D, _ptr(pos), float(alpha), int(window),
                          flags, _ptr(out), _ptr(lse), _stream(stream))
    _check("fsa_decode", st)
    return out, lse


def fsa_rope(x, base, pos0=None, inverse=False, out=None, out_dtype=None,
             stream=None):
    """Rotary position embedding of rows x [B,H,T,D] (fp32 or bf16): row t of
    batch entry b at position pos0[b] + t (pos0: int32 [B] on the device, or
    None for t). inverse=True turns by the negated angles. Returns `out`
    (default: a new tensor of out_dtype, else x's dtype); out may be x itself
    when the dtypes agree."""
    import torch
    if x.dim() != 4 or not x.is_cuda or not x.is_contiguous():
        raise ValueError("x must be a contiguous [B, H, T, D] device tensor")
    B, H, T, D = (int(s) for s in x.shape)
    if out is None:
        out = torch.empty_like(x, dtype=x.dtype if out_dtype is None else out_dtype)
    _need(out, (B, H, T, D), out.dtype, "out")
    if pos0 is not None:
        _need(pos0, (B,), torch.int32, "pos0")
    st = lib().fsa_rope(_ptr(x), _dtype_code(x), B, H, T, D, float(base),
                        _ptr(pos0), int(bool(inverse)), _ptr(out),
                        _dtype_code(out), _stream(stream))
    _check("fsa_rope", st)
    return out


# ------------------------------------------------------------- learned alpha
def _f32_dev(t, n, name):
    import torch
    return _need(t, (n,), torch.float32, name)


def fsa_theta_alpha(theta, theta_map, window, pattern=FSA_PATTERN_FIB, alpha=None,
                    tables=None, stream=None):
    """alpha [L] fp32 and the layers' tap tables (uint8 [L, 256] device
    records) from theta [L] fp32, on the device."""
    import torch
    if not isinstance(theta, torch.Tensor) or theta.dim() != 1:
        raise ValueError("theta must be a 1-D device tensor")
    L = int(theta.shape[0])
    _f32_dev(theta, L, "theta")
    if alpha is None:
        alpha = torch.empty(L, dtype=torch.float32, device=theta.device)
    if tables is None:
        tables = torch.empty((L, FSA_TAP_TABLE_BYTES), dtype=torch.uint8, device=theta.device)
    _f32_dev(alpha, L, "alpha")
    _need(tables, (L, FSA_TAP_TABLE_BYTES), torch.uint8, "tables")
    st = lib().fsa_theta_alpha(_ptr(theta), L, int(theta_map), int(window), int(pattern),
                               _ptr(alpha), _ptr(tables), _stream(stream))
    _check("fsa_theta_alpha", st)
    return alpha, tables


def fsa_theta_step(theta, dalpha, theta_map, optimizer, lr, state, alpha, tables,
                   window, pattern=FSA_PATTERN_FIB, beta1=0.9, beta2=0.999, eps=1e-8,
                   stream=None):
    """One optimizer update of theta [L] from dalpha [L] (device fp32); state is
    a zeroed uint8 device tensor of theta_state_bytes(L) at the first update;
    alpha and tables receive the new alpha and tap tables."""
    import torch
    L = int(theta.shape[0])
    _f32_dev(theta, L, "theta")
    _f32_dev(dalpha, L, "dalpha")
    _f32_dev(alpha, L, "alpha")
    _need(tables, (L, FSA_TAP_TABLE_BYTES), torch.uint8, "tables")
    _need(state, (theta_state_bytes(L),), torch.uint8, "state")
    st = lib().fsa_theta_step(_ptr(theta), _ptr(dalpha), L, int(theta_map), int(optimizer),
                              float(lr), float(beta1), float(beta2), float(eps),
                              _ptr(state), int(window), int(pattern), _ptr(alpha),
                              _ptr(tables), _stream(stream))
    _check("fsa_theta_step", st)


def fsa_forward_dev(q, k, v, table, window, out=None, lse=None, stream=None,
                    out_dtype=None):
    """fsa_forward with the layer's tap table from device memory (a row of the
    tables that fsa_theta_alpha / fsa_theta_step write)."""
    import torch
    B, H, T, D = _shape(q)
    _rows(q, (k, v))
    _need(table, (FSA_TAP_TABLE_BYTES,), torch.uint8, "table")
    out, flags = _out_buffer(out, out_dtype, (B, H, T, D), q.device, 0)
    if lse is None:
        lse = torch.empty((B, H, T), dtype=torch.float32, device=q.device)
    _need(lse, (B, H, T), torch.float32, "lse")
    st = lib().fsa_forward_dev(_ptr(q), _ptr(k), _ptr(v), _dtype_code(q), B, H, T, D,
                               _ptr(table), int(window), flags, _ptr(out), _ptr(lse),
                               _stream(stream))
    _check("fsa_forward_dev", st)
    return out, lse


def fsa_backward_dev(q, k, v, dout, lse, table, window, dq=None, dk=None, dv=None,
                     dalpha=None, workspace=None, stream=None):
    """fsa_backward with the layer's tap table from device memory; dalpha is a
    [1] fp32 device tensor (a view of one layer's slot is fine)."""
    import torch
    B, H, T, D = _shape(q)
    _rows(q, (k, v, dout))
    _need(table, (FSA_TAP_TABLE_BYTES,), torch.uint8, "table")
    dt = _dtype_code(q)
    f32 = torch.float32
    mk = lambda: torch.empty((B, H, T, D), dtype=f32, device=q.device)
    dq = mk() if dq is None else _need(dq, (B, H, T, D), f32, "dq")
    dk = mk() if dk is None else _need(dk, (B, H, T, D), f32, "dk")
    dv = mk() if dv is None else _need(dv, (B, H, T, D), f32, "dv")
    _need(lse, (B, H, T), f32, "lse")
    if dalpha is None:
        dalpha = torch.empty(1, dtype=f32, device=q.device)
    _need(dalpha, (1,), f32, "dalpha")
    nbytes = fsa_backward_workspace_size(B, H, T, D, dt)
    if workspace is None:
        workspace = torch.empty(max(nbytes, 1), dtype=torch.uint8, device=q.device)
    _workspace(workspace, nbytes)
    st = lib().fsa_backward_dev(_ptr(q), _ptr(k), _ptr(v), _ptr(dout), _ptr(lse), dt,
                                B, H, T, D, _ptr(table), int(window), _ptr(dq), _ptr(dk),
                                _ptr(dv), _ptr(dalpha), _ptr(workspace),
                                _ws_bytes(workspace), _stream(stream))
    _check("fsa_backward_dev", st)
    return dq, dk, dv, dalpha


# ------------------------------------------------------------- fused RoPE
def fsa_forward_rope(q_pre, k, v, alpha, window, base, pos0=None, out=None, lse=None,
                     q_rot=None, stream=None, pattern=FSA_PATTERN_FIB, out_dtype=None,
                     want_q_rot=True):
    """fsa_forward with the query rows given before RoPE (bf16): the kernel
    turns each query tile; k must already be rotated. Returns (out, lse,
    q_rot) with q_rot the turned query rows (bf16), or None when
    want_q_rot is False."""
    import torch
    B, H, T, D = _shape(q_pre)
    _rows(q_pre, (k, v))
    out, flags = _out_buffer(out, out_dtype, (B, H, T, D), q_pre.device, pattern)
    if lse is None:
        lse = torch.empty((B, H, T), dtype=torch.float32, device=q_pre.device)
    _need(lse, (B, H, T), torch.float32, "lse")
    if want_q_rot and q_rot is None:
        q_rot = torch.empty_like(q_pre)
    if q_rot is not None:
        _need(q_rot, (B, H, T, D), q_pre.dtype, "q_rot")
    if pos0 is not None:
        _need(pos0, (B,), torch.int32, "pos0")
    st = lib().fsa_forward_rope(_ptr(q_pre), _ptr(k), _ptr(v), _dtype_code(q_pre), B, H,
                                T, D, float(alpha), int(window), flags, float(base),
                                _ptr(pos0), _ptr(out), _ptr(lse), _ptr(q_rot),
                                _stream(stream))
    _check("fsa_forward_rope", st)
    return out, lse, q_rot


def fsa_backward_rope(q, k, v, dout, lse, alpha, window, base, pos0=None, dq=None,
                      dk=None, dv=None, dalpha=None, workspace=None, stream=None,
                      pattern=FSA_PATTERN_FIB):
    """fsa_backward on rotated q, k (bf16), with dq and dk returned as the
    gradients with respect to the rows before rotation."""
    import torch
    B, H, T, D = _shape(q)
    _rows(q, (k, v, dout))
    dt = _dtype_code(q)
    f32 = torch.float32
    mk = lambda: torch.empty((B, H, T, D), dtype=f32, device=q.device)
    dq = mk() if dq is None else _need(dq, (B, H, T, D), f32, "dq")
    dk = mk() if dk is None else _need(dk, (B, H, T, D), f32, "dk")
    dv = mk() if dv is None else _need(dv, (B, H, T, D), f32, "dv")
    _need(lse, (B, H, T), f32, "lse")
    if dalpha is None:
        dalpha = torch.empty(1, dtype=f32, device=q.device)
    _need(dalpha, (1,), f32, "dalpha")
    if pos0 is not None:
        _need(pos0, (B,), torch.int32, "pos0")
    nbytes = fsa_backward_workspace_size(B, H, T, D, dt)
    if workspace is None:
        workspace = torch.empty(max(nbytes, 1), dtype=torch.uint8, device=q.device)
    _workspace(workspace, nbytes)
    st = lib().fsa_backward_rope(_ptr(q), _ptr(k), _ptr(v), _ptr(dout), _ptr(lse), dt,
                                 B, H, T, D, float(alpha), int(window), int(pattern),
                                 float(base), _ptr(pos0), _ptr(dq), _ptr(dk), _ptr(dv),
                                 _ptr(dalpha), _ptr(workspace), _ws_bytes(workspace),
                                 _stream(stream))
    _check("fsa_backward_rope", st)
    return dq, dk, dv, dalpha
