"""ctypes binding of libkda.so (include/kda.h).

Argument marshalling only: tensors are checked for device, dtype, shape and
contiguity, outputs are allocated with torch, and the C entry point is called
on the current HIP stream.  Every step of the computation runs in the HIP
kernels; if the library is missing this module raises -- there is no other
path.
"""
from __future__ import annotations

import ctypes
import os
import threading

PKG = os.path.dirname(os.path.abspath(__file__))
LIBRARY = os.path.join(PKG, "libkda.so")

KDA_F32, KDA_BF16 = 0, 1
ABI_VERSION = 3
STATUS_NAMES = {
    0: "KDA_OK", 1: "KDA_ERR_NULL", 2: "KDA_ERR_SHAPE", 3: "KDA_ERR_DTYPE",
    4: "KDA_ERR_ALIGN", 5: "KDA_ERR_UNSUPPORTED", 6: "KDA_ERR_HIP",
    7: "KDA_ERR_WORKSPACE", 8: "KDA_ERR_PRECONDITION", 9: "KDA_ERR_OVERLAP",
}
# workspace_bytes value asking the library to allocate the workspace itself
KDA_WORKSPACE_AUTO = -1
# prefill plans, fastest first
KDA_PLAN_FULL, KDA_PLAN_SEGMENTS, KDA_PLAN_UNSEGMENTED = 0, 1, 2
EXPORTS = ("kda_prefill", "kda_prefill_noalloc", "kda_varlen_prefill", "kda_decode_step", "kda_prefill_raw",
           "kda_varlen_prefill_raw", "kda_decode_step_raw", "kda_decode_tokens",
           "kda_decode_step_slots", "kda_varlen_prefill_slots", "kda_backward",
           "kda_varlen_backward", "kda_prefill_workspace_size",
           "kda_varlen_prefill_workspace_size", "kda_backward_workspace_size",
           "kda_varlen_backward_workspace_size", "kda_set_prefill_segment", "kda_status_str",
           "kda_abi_version")

_lock = threading.Lock()
_lib = None


class KDAError(RuntimeError):
    """A non-OK kda_status returned by the library."""

    def __init__(self, fn, code, text):
        super().__init__(f"{fn}: {text} (status {code})")
        self.code = code


def load_library(path: str | None = None):
    """Load libkda.so and declare the C signatures.  Raises if it is not built.

    torch is imported first: libkda.so then binds to the HIP runtime that
    torch already loaded, so device memory, streams and the library's own
    runtime calls all go through one runtime.  (Loaded first, the library
    would pull in the system copy and the process would hold two.)"""
    global _lib
    _torch()
    with _lock:
        if _lib is not None and path is None:
            return _lib
        target = path or LIBRARY
        if not os.path.exists(target):
            raise ImportError(
                f"{target} is missing: build the KDA HIP library first "
                "(python -m gated_delta_rule_113_amd.build)")
        lib = ctypes.CDLL(target)
        vp, i64, f32p = ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p
        i64p = ctypes.POINTER(ctypes.c_int64)
        lib.kda_prefill.argtypes = [vp, vp, vp, vp, f32p, f32p, f32p, f32p,
                                    i64, i64, i64, i64, i64, ctypes.c_int, vp, i64, vp]
        lib.kda_prefill.restype = ctypes.c_int
        lib.kda_prefill_noalloc.argtypes = [vp, vp, vp, vp, f32p, f32p, f32p, f32p,
                                            i64, i64, i64, i64, i64, ctypes.c_int, vp]
        lib.kda_prefill_noalloc.restype = ctypes.c_int
        lib.kda_prefill_raw.argtypes = lib.kda_prefill.argtypes
        lib.kda_prefill_raw.restype = ctypes.c_int
        lib.kda_varlen_prefill.argtypes = [vp, vp, vp, vp, f32p, vp, i64, i64,
                                           f32p, f32p, f32p, i64, i64, i64, ctypes.c_int, vp, i64,
                                           vp]
        lib.kda_varlen_prefill.restype = ctypes.c_int
        lib.kda_varlen_prefill_raw.argtypes = lib.kda_varlen_prefill.argtypes
        lib.kda_varlen_prefill_raw.restype = ctypes.c_int
        lib.kda_decode_step.argtypes = [vp, vp, vp, vp, f32p, f32p, f32p,
                                        i64, i64, i64, i64, ctypes.c_int, vp]
        lib.kda_decode_step.restype = ctypes.c_int
        lib.kda_decode_step_raw.argtypes = lib.kda_decode_step.argtypes
        lib.kda_decode_step_raw.restype = ctypes.c_int
        lib.kda_decode_tokens.argtypes = [vp, vp, vp, vp, f32p, f32p, vp, f32p,
                                          i64, i64, i64, i64, i64, ctypes.c_int, vp]
        lib.kda_decode_tokens.restype = ctypes.c_int
        lib.kda_decode_step_slots.argtypes = [vp, vp, vp, vp, f32p, f32p, vp, i64, f32p,
                                              i64, i64, i64, i64, ctypes.c_int, vp]
        lib.kda_decode_step_slots.restype = ctypes.c_int
        lib.kda_varlen_prefill_slots.argtypes = [vp, vp, vp, vp, f32p, vp, i64, i64, f32p, vp, vp,
                                                 i64, f32p, i64, i64, i64, ctypes.c_int, vp, i64,
                                                 vp]
        lib.kda_varlen_prefill_slots.restype = ctypes.c_int
        lib.kda_backward.argtypes = [vp, vp, vp, vp, f32p, f32p, f32p, f32p,
                                     f32p, f32p, f32p, f32p, f32p, f32p,
                                     i64, i64, i64, i64, i64, ctypes.c_int, vp, i64, vp]
        lib.kda_backward.restype = ctypes.c_int
        lib.kda_varlen_backward.argtypes = [vp, vp, vp, vp, f32p, vp, i64, i64, f32p, f32p, f32p,
                                            f32p, f32p, f32p, f32p, f32p, f32p,
                                            i64, i64, i64, ctypes.c_int, vp, i64, vp]
        lib.kda_varlen_backward.restype = ctypes.c_int
        lib.kda_set_prefill_segment.argtypes = [i64]
        lib.kda_set_prefill_segment.restype = ctypes.c_int
        lib.kda_prefill_workspace_size.argtypes = [i64, i64, i64, i64, i64, ctypes.c_int,
                                                   ctypes.c_int, i64p]
        lib.kda_prefill_workspace_size.restype = ctypes.c_int
        lib.kda_varlen_prefill_workspace_size.argtypes = lib.kda_prefill_workspace_size.argtypes
        lib.kda_varlen_prefill_workspace_size.restype = ctypes.c_int
        lib.kda_backward_workspace_size.argtypes = [i64, i64, i64, i64, i64, ctypes.c_int, i64p]
        lib.kda_backward_workspace_size.restype = ctypes.c_int
        lib.kda_varlen_backward_workspace_size.argtypes = lib.kda_backward_workspace_size.argtypes
        lib.kda_varlen_backward_workspace_size.restype = ctypes.c_int
        lib.kda_status_str.argtypes = [ctypes.c_int]
        lib.kda_status_str.restype = ctypes.c_char_p
        lib.kda_abi_version.argtypes = []
        lib.kda_abi_version.restype = ctypes.c_int
        if lib.kda_abi_version() != ABI_VERSION:
            raise ImportError(f"{target} implements ABI {lib.kda_abi_version()}, this binding "
                              f"ABI {ABI_VERSION}: rebuild the library")
        if path is None:
            _lib = lib
        return lib


def _check(lib, fn, code):
    if code != 0:
        raise KDAError(fn, code, lib.kda_status_str(code).decode())


def _torch():
    import torch
    return torch


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _on(device):
    """The library allocates its workspace on, and counts the compute units
    of, the calling thread's current device: make it the tensors' device."""
    return _torch().cuda.device(device)


def _stream(device):
    torch = _torch()
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _size_query(lib, fn, *args):
    """A *_workspace_size call: the bytes it reports."""
    out = ctypes.c_int64(0)
    _check(lib, fn, getattr(lib, fn)(*args, ctypes.byref(out)))
    return int(out.value)


def _workspace(workspace, size, dev):
    """(pointer, bytes, keep-alive) for a call's workspace argument.

    None: a torch tensor of the fastest plan's size (``size()``), allocated by
    torch's caching allocator on the current stream (stream-ordered, so it may
    be dropped once the call is enqueued); "auto": KDA_WORKSPACE_AUTO (the
    library allocates); a tensor: its bytes, caller-owned."""
    torch = _torch()
    if workspace is None:
        n = size()
        if n == 0:
            return None, 0, None
        t = torch.empty(n, dtype=torch.uint8, device=dev)
        return _ptr(t), n, t
    if isinstance(workspace, str):
        if workspace != "auto":
            raise ValueError('workspace must be None, "auto" or a tensor')
        return None, KDA_WORKSPACE_AUTO, None
    _require(workspace, "workspace", device=dev)
    return _ptr(workspace), workspace.numel() * workspace.element_size(), workspace


def prefill_workspace_size(B, T, H, dtype, plan=KDA_PLAN_FULL, device=None, d=128):
    """Bytes of workspace kda_prefill needs for [B, T, H, d] inputs of torch
    dtype ``dtype`` under ``plan`` on ``device`` (default: the current one)."""
    lib = load_library()
    with _on(device if device is not None else _torch().cuda.current_device()):
        return _size_query(lib, "kda_prefill_workspace_size", B, T, H, d, d,
                           _dtype_code(dtype), plan)


def varlen_prefill_workspace_size(N, T_total, H, dtype, plan=KDA_PLAN_FULL, device=None, d=128):
    """Bytes of workspace kda_varlen_prefill needs for N packed sequences of
    T_total rows in all (see prefill_workspace_size)."""
    lib = load_library()
    with _on(device if device is not None else _torch().cuda.current_device()):
        return _size_query(lib, "kda_varlen_prefill_workspace_size", N, T_total, H, d, d,
                           _dtype_code(dtype), plan)


def backward_workspace_size(B, T, H, dtype, device=None, d=128, cu_seqlens_n=None):
    """Bytes of workspace kda_backward needs for [B, T, H, d] inputs (or, with
    ``cu_seqlens_n`` = N, kda_varlen_backward for N sequences of T rows in all)."""
    lib = load_library()
    with _on(device if device is not None else _torch().cuda.current_device()):
        if cu_seqlens_n is None:
            return _size_query(lib, "kda_backward_workspace_size", B, T, H, d, d, _dtype_code(dtype))
        return _size_query(lib, "kda_varlen_backward_workspace_size", cu_seqlens_n, T, H, d, d,
                           _dtype_code(dtype))


def _dtype_code(dt):
    torch = _torch()
    if dt == torch.float32:
        return KDA_F32
    if dt == torch.bfloat16:
        return KDA_BF16
    raise TypeError(f"q, k, v, beta must be float32 or bfloat16, got {dt}")


def _in_dtype(*ts):
    torch = _torch()
    dt = ts[0].dtype
    for t in ts:
        if t.dtype != dt:
            raise TypeError("q, k, v and beta must share one dtype")
    if dt == torch.float32:
        return KDA_F32
    if dt == torch.bfloat16:
        return KDA_BF16
    raise TypeError(f"q, k, v, beta must be float32 or bfloat16, got {dt}")


def _require(t, name, dtype=None, shape=None, device=None):
    torch = _torch()
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if not t.is_cuda:
        raise ValueError(f"{name} must be on the GPU")
    if device is not None and t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return t


def kda_prefill(q, k, v, beta, log_alpha, initial_state=None, *, out=None, final_state=None,
                workspace=None, _fn="kda_prefill"):
    """Dense prefill.  q, k, log_alpha [B, T, H, 128]; v [B, T, H, 128];
    beta [B, T, H]; initial_state [B, H, 128, 128] fp32 or None.

    Returns (o [B, T, H, 128] fp32, final_state [B, H, 128, 128] fp32).
    ``final_state`` may be passed (and may be ``initial_state``) to write in place.
    ``workspace``: None (a torch tensor of the fastest plan's size), "auto"
    (the library allocates) or a caller-owned device tensor (its bytes pick
    the plan).
    """
    torch = _torch()
    lib = load_library()
    B, T, H, dk = q.shape
    dv = v.shape[-1]
    dev = q.device
    _require(q, "q", device=dev)
    _require(k, "k", q.dtype, (B, T, H, dk), dev)
    _require(v, "v", q.dtype, (B, T, H, dv), dev)
    _require(beta, "beta", q.dtype, (B, T, H), dev)
    _require(log_alpha, "log_alpha", torch.float32, (B, T, H, dk), dev)
    if initial_state is not None:
        _require(initial_state, "initial_state", torch.float32, (B, H, dk, dv), dev)
    o = out if out is not None else torch.empty((B, T, H, dv), dtype=torch.float32, device=dev)
    _require(o, "out", torch.float32, (B, T, H, dv), dev)
    if final_state is None:
        final_state = torch.empty((B, H, dk, dv), dtype=torch.float32, device=dev)
    _require(final_state, "final_state", torch.float32, (B, H, dk, dv), dev)
    dt = _in_dtype(q, k, v, beta)
    with _on(dev):
        wp, wb, _keep = _workspace(workspace, lambda: _size_query(
            lib, "kda_prefill_workspace_size", B, T, H, dk, dv, dt, KDA_PLAN_FULL), dev)
        code = getattr(lib, _fn)(_ptr(q), _ptr(k), _ptr(v), _ptr(beta), _ptr(log_alpha),
                                 _ptr(initial_state), _ptr(o), _ptr(final_state),
                                 B, T, H, dk, dv, dt, wp, wb, _stream(dev))
    _check(lib, _fn, code)
    return o, final_state


def kda_varlen_prefill(q, k, v, beta, log_alpha, cu_seqlens, initial_state=None, *,
                       out=None, final_state=None, workspace=None, _fn="kda_varlen_prefill"):
    """Packed prefill.  q, k, log_alpha [1, T_total, H, 128] (or [T_total, H, 128]);
    cu_seqlens int32 [N + 1] on the GPU; initial_state [N, H, 128, 128] or None.

    Returns (o shaped like v but fp32, final_state [N, H, 128, 128] fp32).
    ``workspace`` as in kda_prefill.
    """
    torch = _torch()
    lib = load_library()
    dev = q.device
    lead = q.shape[:-3]
    if lead not in ((), (1,)):
        raise ValueError("packed inputs must be [T_total, H, d] or [1, T_total, H, d]")
    Tt, H, dk = q.shape[-3:]
    dv = v.shape[-1]
    _require(q, "q", device=dev)
    _require(k, "k", q.dtype, (*lead, Tt, H, dk), dev)
    _require(v, "v", q.dtype, (*lead, Tt, H, dv), dev)
    _require(beta, "beta", q.dtype, (*lead, Tt, H), dev)
    _require(log_alpha, "log_alpha", torch.float32, (*lead, Tt, H, dk), dev)
    _require(cu_seqlens, "cu_seqlens", torch.int32, None, dev)
    if cu_seqlens.dim() != 1 or cu_seqlens.numel() < 1:
        raise ValueError("cu_seqlens must be a 1-D int32 tensor of N + 1 offsets")
    N = cu_seqlens.numel() - 1
    if initial_state is not None:
        _require(initial_state, "initial_state", torch.float32, (N, H, dk, dv), dev)
    o = out if out is not None else torch.empty((*lead, Tt, H, dv), dtype=torch.float32, device=dev)
    _require(o, "out", torch.float32, (*lead, Tt, H, dv), dev)
    if final_state is None:
        final_state = torch.empty((N, H, dk, dv), dtype=torch.float32, device=dev)
    _require(final_state, "final_state", torch.float32, (N, H, dk, dv), dev)
    dt = _in_dtype(q, k, v, beta)
    with _on(dev):
        wp, wb, _keep = _workspace(workspace, lambda: _size_query(
            lib, "kda_varlen_prefill_workspace_size", N, Tt, H, dk, dv, dt, KDA_PLAN_FULL), dev)
        code = getattr(lib, _fn)(_ptr(q), _ptr(k), _ptr(v), _ptr(beta), _ptr(log_alpha),
                                 _ptr(cu_seqlens), N, Tt, _ptr(initial_state), _ptr(o),
                                 _ptr(final_state), H, dk, dv, dt, wp, wb, _stream(dev))
    _check(lib, _fn, code)
    return o, final_state


def _backward(q, k, v, beta, log_alpha, d_o, cu_seqlens, initial_state, d_final_state, workspace):
    """Shared marshalling of kda_backward / kda_varlen_backward."""
    torch = _torch()
    lib = load_library()
    dev = q.device
    rows = tuple(q.shape[:-2])
    H, dk = q.shape[-2:]
    dv = v.shape[-1]
    _require(q, "q", device=dev)
    _require(k, "k", q.dtype, (*rows, H, dk), dev)
    _require(v, "v", q.dtype, (*rows, H, dv), dev)
    _require(beta, "beta", q.dtype, (*rows, H), dev)
    _require(log_alpha, "log_alpha", torch.float32, (*rows, H, dk), dev)
    _require(d_o, "d_o", torch.float32, (*rows, H, dv), dev)
    if cu_seqlens is None:
        B, T = rows
        units = B
    else:
        if rows[:-1] not in ((), (1,)):
            raise ValueError("packed inputs must be [T_total, H, d] or [1, T_total, H, d]")
        _require(cu_seqlens, "cu_seqlens", torch.int32, None, dev)
        if cu_seqlens.dim() != 1 or cu_seqlens.numel() < 1:
            raise ValueError("cu_seqlens must be a 1-D int32 tensor of N + 1 offsets")
        units = cu_seqlens.numel() - 1
        Tt = rows[-1]
    sshape = (units, H, dk, dv)
    if initial_state is not None:
        _require(initial_state, "initial_state", torch.float32, sshape, dev)
    if d_final_state is not None:
        _require(d_final_state, "d_final_state", torch.float32, sshape, dev)
    g = {name: torch.empty(like.shape, dtype=torch.float32, device=dev)
         for name, like in (("dq", q), ("dk", k), ("dv", v), ("dbeta", beta),
                            ("dlog_alpha", log_alpha))}
    g["dinitial_state"] = torch.empty(sshape, dtype=torch.float32, device=dev)
    dt = _in_dtype(q, k, v, beta)
    with _on(dev):
        if cu_seqlens is None:
            fn = "kda_backward"
            wp, wb, _keep = _workspace(workspace, lambda: _size_query(
                lib, "kda_backward_workspace_size", B, T, H, dk, dv, dt), dev)
            code = lib.kda_backward(_ptr(q), _ptr(k), _ptr(v), _ptr(beta), _ptr(log_alpha),
                                    _ptr(initial_state), _ptr(d_o), _ptr(d_final_state),
                                    _ptr(g["dq"]), _ptr(g["dk"]), _ptr(g["dv"]), _ptr(g["dbeta"]),
                                    _ptr(g["dlog_alpha"]), _ptr(g["dinitial_state"]),
                                    B, T, H, dk, dv, dt, wp, wb, _stream(dev))
        else:
            fn = "kda_varlen_backward"
            wp, wb, _keep = _workspace(workspace, lambda: _size_query(
                lib, "kda_varlen_backward_workspace_size", units, Tt, H, dk, dv, dt), dev)
            code = lib.kda_varlen_backward(_ptr(q), _ptr(k), _ptr(v), _ptr(beta), _ptr(log_alpha),
                                           _ptr(cu_seqlens), units, Tt, _ptr(initial_state),
                                           _ptr(d_o), _ptr(d_final_state), _ptr(g["dq"]),
                                           _ptr(g["dk"]), _ptr(g["dv"]), _ptr(g["dbeta"]),
                                           _ptr(g["dlog_alpha"]), _ptr(g["dinitial_state"]),
                                           H, dk, dv, dt, wp, wb, _stream(dev))
    _check(lib, fn, code)
    return g


def kda_backward(q, k, v, beta, log_alpha, d_o, initial_state=None, d_final_state=None, *,
                 workspace=None):
    """Gradients of a dense prefill.  Inputs as kda_prefill, plus d_o (fp32,
    shaped like o) and d_final_state ([B, H, 128, 128] fp32 or None = zeros).

    Returns a dict of fp32 tensors: dq, dk, dv, dbeta, dlog_alpha (each shaped
    like its input) and dinitial_state [B, H, 128, 128].  ``workspace`` as in
    kda_prefill (a caller-owned one must hold kda_backward_workspace_size bytes).
    """
    if q.dim() != 4:
        raise ValueError("dense inputs must be [B, T, H, d]")
    return _backward(q, k, v, beta, log_alpha, d_o, None, initial_state, d_final_state, workspace)


def kda_varlen_backward(q, k, v, beta, log_alpha, d_o, cu_seqlens, initial_state=None,
                        d_final_state=None, *, workspace=None):
    """Gradients of a packed prefill (inputs as kda_varlen_prefill, plus d_o
    and d_final_state [N, H, 128, 128] or None).  Returns the dict of
    kda_backward, dinitial_state [N, H, 128, 128]."""
    return _backward(q, k, v, beta, log_alpha, d_o, cu_seqlens, initial_state, d_final_state,
                     workspace)


def kda_set_prefill_segment(tokens: int) -> None:
    """Force the prefill segment length (a multiple of 64), or 0 for automatic."""
    lib = load_library()
    _check(lib, "kda_set_prefill_segment", lib.kda_set_prefill_segment(int(tokens)))


def kda_decode_step(q, k, v, beta, log_alpha, state, *, out=None, _fn="kda_decode_step"):
    """One decode step.  q, k, log_alpha [N, H, 128]; v [N, H, 128]; beta [N, H];
    state [N, H, 128, 128] fp32, updated in place.  Returns o [N, H, 128] fp32."""
    torch = _torch()
    lib = load_library()
    N, H, dk = q.shape
    dv = v.shape[-1]
    dev = q.device
    _require(q, "q", device=dev)
    _require(k, "k", q.dtype, (N, H, dk), dev)
    _require(v, "v", q.dtype, (N, H, dv), dev)
    _require(beta, "beta", q.dtype, (N, H), dev)
    _require(log_alpha, "log_alpha", torch.float32, (N, H, dk), dev)
    _require(state, "state", torch.float32, (N, H, dk, dv), dev)
    o = out if out is not None else torch.empty((N, H, dv), dtype=torch.float32, device=dev)
    _require(o, "out", torch.float32, (N, H, dv), dev)
    with _on(dev):
        code = getattr(lib, _fn)(_ptr(q), _ptr(k), _ptr(v), _ptr(beta), _ptr(log_alpha),
                                 _ptr(state), _ptr(o), N, H, dk, dv, _in_dtype(q, k, v, beta),
                                 _stream(dev))
    _check(lib, _fn, code)
    return o


def _slots(t, name, N, dev):
    torch = _torch()
    _require(t, name, torch.int32, (N,), dev)
    return t


def kda_decode_step_slots(q, k, v, beta, log_alpha, state_pool, slots, *, out=None):
    """One decode step with the states in a pool.  q, k, log_alpha [N, H, 128];
    v [N, H, 128]; beta [N, H]; state_pool [P, H, 128, 128] fp32; slots int32 [N]
    on the GPU.  Sequence n updates pool entry slots[n] in place; a slot outside
    [0, P) skips the sequence (its rows of ``out`` are left as they are; without
    ``out`` they are zeros).  Returns o [N, H, 128] fp32."""
    torch = _torch()
    lib = load_library()
    N, H, dk = q.shape
    dv = v.shape[-1]
    dev = q.device
    _require(q, "q", device=dev)
    _require(k, "k", q.dtype, (N, H, dk), dev)
    _require(v, "v", q.dtype, (N, H, dv), dev)
    _require(beta, "beta", q.dtype, (N, H), dev)
    _require(log_alpha, "log_alpha", torch.float32, (N, H, dk), dev)
    _require(state_pool, "state_pool", torch.float32, None, dev)
    if state_pool.dim() != 4 or tuple(state_pool.shape[1:]) != (H, dk, dv):
        raise ValueError(f"state_pool must be [P, {H}, {dk}, {dv}], got {tuple(state_pool.shape)}")
    _slots(slots, "slots", N, dev)
    o = out if out is not None else torch.zeros((N, H, dv), dtype=torch.float32, device=dev)
    _require(o, "out", torch.float32, (N, H, dv), dev)
    with _on(dev):
        code = lib.kda_decode_step_slots(_ptr(q), _ptr(k), _ptr(v), _ptr(beta), _ptr(log_alpha),
                                         _ptr(state_pool), _ptr(slots), state_pool.shape[0], _ptr(o),
                                         N, H, dk, dv, _in_dtype(q, k, v, beta), _stream(dev))
    _check(lib, "kda_decode_step_slots", code)
    return o


def kda_varlen_prefill_slots(q, k, v, beta, log_alpha, cu_seqlens, state_pool, init_slots=None,
                             final_slots=None, *, out=None, workspace=None):
    """Packed prefill with the states in a pool.  Inputs as kda_varlen_prefill;
    state_pool [P, H, 128, 128] fp32; init_slots / final_slots int32 [N] on the
    GPU or None.  Sequence n starts from pool entry init_slots[n] (zeros when
    outside [0, P) or when init_slots is None) and leaves its final state in pool
    entry final_slots[n] (not written when outside [0, P) or when final_slots is
    None).  Returns o shaped like v, fp32."""
    torch = _torch()
    lib = load_library()
    dev = q.device
    lead = q.shape[:-3]
    if lead not in ((), (1,)):
        raise ValueError("packed inputs must be [T_total, H, d] or [1, T_total, H, d]")
    Tt, H, dk = q.shape[-3:]
    dv = v.shape[-1]
    _require(q, "q", device=dev)
    _require(k, "k", q.dtype, (*lead, Tt, H, dk), dev)
    _require(v, "v", q.dtype, (*lead, Tt, H, dv), dev)
    _require(beta, "beta", q.dtype, (*lead, Tt, H), dev)
    _require(log_alpha, "log_alpha", torch.float32, (*lead, Tt, H, dk), dev)
    _require(cu_seqlens, "cu_seqlens", torch.int32, None, dev)
    if cu_seqlens.dim() != 1 or cu_seqlens.numel() < 1:
        raise ValueError("cu_seqlens must be a 1-D int32 tensor of N + 1 offsets")
    N = cu_seqlens.numel() - 1
    _require(state_pool, "state_pool", torch.float32, None, dev)
    if state_pool.dim() != 4 or tuple(state_pool.shape[1:]) != (H, dk, dv):
        raise ValueError(f"state_pool must be [P, {H}, {dk}, {dv}], got {tuple(state_pool.shape)}")
    if init_slots is not None:
        _slots(init_slots, "init_slots", N, dev)
    if final_slots is not None:
        _slots(final_slots, "final_slots", N, dev)
    o = out if out is not None else torch.empty((*lead, Tt, H, dv), dtype=torch.float32, device=dev)
    _require(o, "out", torch.float32, (*lead, Tt, H, dv), dev)
    dt = _in_dtype(q, k, v, beta)
    with _on(dev):
        wp, wb, _keep = _workspace(workspace, lambda: _size_query(
            lib, "kda_varlen_prefill_workspace_size", N, Tt, H, dk, dv, dt, KDA_PLAN_FULL), dev)
        code = lib.kda_varlen_prefill_slots(_ptr(q), _ptr(k), _ptr(v), _ptr(beta), _ptr(log_alpha),
                                            _ptr(cu_seqlens), N, Tt, _ptr(state_pool),
                                            _ptr(init_slots), _ptr(final_slots), state_pool.shape[0],
                                            _ptr(o), H, dk, dv, dt, wp, wb, _stream(dev))
    _check(lib, "kda_varlen_prefill_slots", code)
    return o


def kda_decode_tokens(q, k, v, beta, log_alpha, state, n_commit=None, *, out=None):
    """K draft tokens per sequence from its state (1 <= K <= 16).  q, k, log_alpha
    [N, K, H, 128]; v [N, K, H, 128]; beta [N, K, H]; state [N, H, 128, 128] fp32.
    Without ``n_commit`` the state is only read; with ``n_commit`` (int32 [N] on
    the GPU) sequence n's state becomes, in place, the state after its first
    n_commit[n] tokens (clamped to [0, K]).  Returns o [N, K, H, 128] fp32."""
    torch = _torch()
    lib = load_library()
    N, K, H, dk = q.shape
    dv = v.shape[-1]
    dev = q.device
    _require(q, "q", device=dev)
    _require(k, "k", q.dtype, (N, K, H, dk), dev)
    _require(v, "v", q.dtype, (N, K, H, dv), dev)
    _require(beta, "beta", q.dtype, (N, K, H), dev)
    _require(log_alpha, "log_alpha", torch.float32, (N, K, H, dk), dev)
    _require(state, "state", torch.float32, (N, H, dk, dv), dev)
    if n_commit is not None:
        _slots(n_commit, "n_commit", N, dev)
    o = out if out is not None else torch.empty((N, K, H, dv), dtype=torch.float32, device=dev)
    _require(o, "out", torch.float32, (N, K, H, dv), dev)
    with _on(dev):
        code = lib.kda_decode_tokens(_ptr(q), _ptr(k), _ptr(v), _ptr(beta), _ptr(log_alpha),
                                     _ptr(state), _ptr(n_commit), _ptr(o), N, K, H, dk, dv,
                                     _in_dtype(q, k, v, beta), _stream(dev))
    _check(lib, "kda_decode_tokens", code)
    return o


def kda_prefill_raw(q, k, v, beta, log_alpha, initial_state=None, *, out=None, final_state=None,
                    workspace=None):
    """kda_prefill on raw projections: q and k are normalised per (token, head)
    inside the kernels (and rounded to bf16 for bf16 inputs), ``beta`` holds
    logits (write strength sigmoid(beta)) and ``log_alpha`` gate logits a
    (log forgetting factor -softplus(a))."""
    return kda_prefill(q, k, v, beta, log_alpha, initial_state, out=out, final_state=final_state,
                       workspace=workspace, _fn="kda_prefill_raw")


def kda_varlen_prefill_raw(q, k, v, beta, log_alpha, cu_seqlens, initial_state=None, *, out=None,
                           final_state=None, workspace=None):
    """kda_varlen_prefill on raw projections (see kda_prefill_raw)."""
    return kda_varlen_prefill(q, k, v, beta, log_alpha, cu_seqlens, initial_state, out=out,
                              final_state=final_state, workspace=workspace,
                              _fn="kda_varlen_prefill_raw")


def kda_decode_step_raw(q, k, v, beta, log_alpha, state, *, out=None):
    """kda_decode_step on raw projections (see kda_prefill_raw)."""
    return kda_decode_step(q, k, v, beta, log_alpha, state, out=out, _fn="kda_decode_step_raw")
