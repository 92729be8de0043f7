"""KDA reference oracle -- TEST INFRASTRUCTURE ONLY.

A ctypes wrapper around ``kda_oracle.c``: the plain fp64, token-by-token
evaluation of Kimi Delta Attention (the channel-wise gated delta rule).
Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this package.  The GPU library never imports it and
shares no code with it: the two meet only on the seeded inputs produced by
``kda_inputs``.

The recurrence (for each sequence n and head h, see ``kda_oracle.c``):

    S_t = (I - beta_t k_t k_t^T) Diag(alpha_t) S_{t-1} + beta_t k_t v_t^T
    o_t = S_t^T q_t,    alpha_t = exp(log_alpha_t)

taken from "Kimi K3 -- the architecture and infrastructure, explained"
(sections "How the delta rule actually works" and "Kimi Delta Attention: the
load-bearing choice") and "Inside Kimi K3: How Moonshot AI Built the Largest
Open-Source Model" (section "Technical Details").

All results are float64 numpy arrays.  Inputs may be any float dtype that
widens exactly to float32 (float32 itself, or bfloat16 values already widened
to float32 by ``kda_inputs.bf16_to_f32``).
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import threading

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
SOURCE = os.path.join(_HERE, "kda_oracle.c")
LIBRARY = os.path.join(_HERE, "_kda_oracle.so")

_lock = threading.Lock()
_lib = None


def build(source: str = SOURCE, output: str = LIBRARY) -> str:
    """Compile the oracle with gcc (plain -O2, OpenMP across units only)."""
    tmp = output + ".tmp%d" % os.getpid()
    cmd = ["gcc", "-O2", "-fopenmp", "-shared", "-fPIC", "-std=c99",
           "-o", tmp, source, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, output)
    return output


def load(path: str | None = None):
    """Load (building first if needed) and return the ctypes library."""
    global _lib
    with _lock:
        if path is None and _lib is not None:
            return _lib
        target = path or LIBRARY
        if path is None and (not os.path.exists(target)
                             or os.path.getmtime(target) < os.path.getmtime(SOURCE)):
            build()
        lib = ctypes.CDLL(target)
        i64p = ctypes.POINTER(ctypes.c_int64)
        fp = ctypes.POINTER(ctypes.c_float)
        dp = ctypes.POINTER(ctypes.c_double)
        lib.kda_oracle_run.argtypes = [
            ctypes.c_int64, i64p, i64p, ctypes.c_int64,
            ctypes.c_int64, ctypes.c_int64, ctypes.c_int64,
            fp, fp, fp, fp, fp, dp, dp, dp, dp, ctypes.c_int]
        lib.kda_oracle_run.restype = ctypes.c_int
        lib.kda_oracle_prepare.argtypes = [ctypes.c_int64, ctypes.c_int64, ctypes.c_int64,
                                           fp, fp, fp, fp, ctypes.c_int, fp, fp, fp, fp]
        lib.kda_oracle_prepare.restype = ctypes.c_int
        lib.kda_oracle_backward.argtypes = [
            ctypes.c_int64, i64p, i64p, ctypes.c_int64,
            ctypes.c_int64, ctypes.c_int64, ctypes.c_int64,
            fp, fp, fp, fp, fp, dp, dp, dp, dp, dp, dp, dp, dp, dp, ctypes.c_int]
        lib.kda_oracle_backward.restype = ctypes.c_int
        lib.kda_oracle_max_threads.argtypes = [ctypes.c_int]
        lib.kda_oracle_max_threads.restype = ctypes.c_int
        if path is None:
            _lib = lib
        return lib


def _f32(x, name):
    a = np.asarray(x)
    if a.dtype != np.float32:
        if a.dtype not in (np.float64, np.float16):
            raise TypeError(f"{name}: expected a float array, got {a.dtype}")
        b = a.astype(np.float32)
        if not np.array_equal(b.astype(a.dtype), a, equal_nan=True):
            raise ValueError(f"{name}: values are not exactly representable in float32")
        a = b
    return np.ascontiguousarray(a)


def _ptr(a, ctype):
    return a.ctypes.data_as(ctypes.POINTER(ctype))


def run_rows(q, k, v, beta, log_alpha, row0, length, row_step, initial_state=None,
             n_threads: int = 0, lib=None, with_magnitude: bool = False):
    """Core call on token-row addressing.

    q, k, log_alpha: [rows, H, dk]; v: [rows, H, dv]; beta: [rows, H].
    Token t of sequence n is row ``row0[n] + t * row_step``.
    Returns (o [rows, H, dv] float64 -- NaN where no token was visited,
    final_state [n_seq, H, dk, dv] float64), and with ``with_magnitude`` also
    m [rows, H, dv] = |S_t|^T |q_t|, the magnitude of each read-out's terms.
    """
    lib = lib or load()
    q = _f32(q, "q"); k = _f32(k, "k"); v = _f32(v, "v")
    beta = _f32(beta, "beta"); log_alpha = _f32(log_alpha, "log_alpha")
    rows, H, dk = q.shape
    dv = v.shape[2]
    if k.shape != (rows, H, dk) or log_alpha.shape != (rows, H, dk):
        raise ValueError("q, k, log_alpha must share [rows, H, dk]")
    if v.shape[:2] != (rows, H) or beta.shape != (rows, H):
        raise ValueError("v must be [rows, H, dv] and beta [rows, H]")
    row0 = np.ascontiguousarray(row0, dtype=np.int64)
    length = np.ascontiguousarray(length, dtype=np.int64)
    n_seq = row0.shape[0]
    if length.shape != (n_seq,):
        raise ValueError("row0 and length must have the same size")
    for n in range(n_seq):
        if length[n] > 0:
            last = row0[n] + (length[n] - 1) * row_step
            if row0[n] < 0 or last >= rows or last < 0:
                raise ValueError(f"sequence {n} addresses rows outside [0, {rows})")
    s0p = None
    if initial_state is not None:
        s0 = np.ascontiguousarray(initial_state, dtype=np.float64)
        if s0.shape != (n_seq, H, dk, dv):
            raise ValueError(f"initial_state must be {(n_seq, H, dk, dv)}")
        s0p = _ptr(s0, ctypes.c_double)
    o = np.full((rows, H, dv), np.nan, dtype=np.float64)
    mag = np.full((rows, H, dv), np.nan, dtype=np.float64) if with_magnitude else None
    s_final = np.empty((n_seq, H, dk, dv), dtype=np.float64)
    rc = lib.kda_oracle_run(n_seq, _ptr(row0, ctypes.c_int64), _ptr(length, ctypes.c_int64),
                            int(row_step), H, dk, dv,
                            _ptr(q, ctypes.c_float), _ptr(k, ctypes.c_float),
                            _ptr(v, ctypes.c_float), _ptr(beta, ctypes.c_float),
                            _ptr(log_alpha, ctypes.c_float), s0p,
                            _ptr(o, ctypes.c_double),
                            None if mag is None else _ptr(mag, ctypes.c_double),
                            _ptr(s_final, ctypes.c_double), int(n_threads))
    if rc != 0:
        raise RuntimeError(f"kda_oracle_run failed with code {rc}")
    return (o, s_final, mag) if with_magnitude else (o, s_final)


def prefill(q, k, v, beta, log_alpha, initial_state=None, n_threads: int = 0, lib=None,
            with_magnitude: bool = False):
    """Dense batch: q, k, log_alpha [B, T, H, dk]; v [B, T, H, dv]; beta [B, T, H].

    Returns (o [B, T, H, dv], final_state [B, H, dk, dv]), float64 (with
    ``with_magnitude`` also the read-out magnitudes, shaped like o).
    """
    q = np.asarray(q)
    B, T, H, dk = q.shape
    dv = np.asarray(v).shape[-1]
    row0 = np.arange(B, dtype=np.int64) * T
    length = np.full(B, T, dtype=np.int64)
    r = run_rows(np.reshape(q, (B * T, H, dk)), np.reshape(k, (B * T, H, dk)),
                 np.reshape(v, (B * T, H, dv)), np.reshape(beta, (B * T, H)),
                 np.reshape(log_alpha, (B * T, H, dk)), row0, length, 1,
                 initial_state, n_threads, lib, with_magnitude)
    if with_magnitude:
        return r[0].reshape(B, T, H, dv), r[1], r[2].reshape(B, T, H, dv)
    return r[0].reshape(B, T, H, dv), r[1]


def _backward_rows(q, k, v, beta, log_alpha, d_o, row0, length, initial_state, d_final_state,
                   n_threads, lib):
    """kda_oracle_backward on rows [rows, H, *]; sequence n owns rows
    row0[n] .. row0[n]+length[n]-1.  Rows outside every sequence get zeros."""
    lib = lib or load()
    rows, H, dk = np.asarray(q).shape
    dv = np.asarray(v).shape[-1]
    n_seq = len(row0)
    qf = _f32(q, "q"); kf = _f32(k, "k"); vf = _f32(v, "v")
    bf = _f32(beta, "beta"); lf = _f32(log_alpha, "log_alpha")
    do = np.ascontiguousarray(d_o, dtype=np.float64)
    row0 = np.ascontiguousarray(row0, dtype=np.int64)
    length = np.ascontiguousarray(length, dtype=np.int64)
    s0p = dsp = None
    if initial_state is not None:
        s0 = np.ascontiguousarray(initial_state, dtype=np.float64)
        if s0.shape != (n_seq, H, dk, dv):
            raise ValueError(f"initial_state must be {(n_seq, H, dk, dv)}")
        s0p = _ptr(s0, ctypes.c_double)
    if d_final_state is not None:
        ds = np.ascontiguousarray(d_final_state, dtype=np.float64)
        if ds.shape != (n_seq, H, dk, dv):
            raise ValueError(f"d_final_state must be {(n_seq, H, dk, dv)}")
        dsp = _ptr(ds, ctypes.c_double)
    out = {"dq": np.zeros((rows, H, dk)), "dk": np.zeros((rows, H, dk)),
           "dv": np.zeros((rows, H, dv)), "dbeta": np.zeros((rows, H)),
           "dlog_alpha": np.zeros((rows, H, dk)), "dinitial_state": np.zeros((n_seq, H, dk, dv))}
    rc = lib.kda_oracle_backward(n_seq, _ptr(row0, ctypes.c_int64), _ptr(length, ctypes.c_int64),
                                 1, H, dk, dv, _ptr(qf, ctypes.c_float), _ptr(kf, ctypes.c_float),
                                 _ptr(vf, ctypes.c_float), _ptr(bf, ctypes.c_float),
                                 _ptr(lf, ctypes.c_float), s0p, _ptr(do, ctypes.c_double), dsp,
                                 *(_ptr(out[n], ctypes.c_double) for n in
                                   ("dq", "dk", "dv", "dbeta", "dlog_alpha", "dinitial_state")),
                                 int(n_threads))
    if rc != 0:
        raise RuntimeError(f"kda_oracle_backward failed with code {rc}")
    return out


def backward(q, k, v, beta, log_alpha, d_o, initial_state=None, d_final_state=None,
             n_threads: int = 0, lib=None):
    """Gradients of L = sum <d_o, o> + <d_final_state, final_state> for a dense
    batch (shapes as in ``prefill``; d_o like o, d_final_state like the final
    state), by the chain rule through the token recurrence in reverse
    (``kda_oracle_backward``).  Returns a dict of float64 arrays: dq, dk, dv,
    dbeta, dlog_alpha (shaped like their inputs) and dinitial_state
    [B, H, dk, dv].  The reference for the library's backward pass."""
    q = np.asarray(q)
    B, T, H, dk = q.shape
    dv = np.asarray(v).shape[-1]
    rows = B * T
    out = _backward_rows(np.reshape(q, (rows, H, dk)), np.reshape(k, (rows, H, dk)),
                         np.reshape(v, (rows, H, dv)), np.reshape(beta, (rows, H)),
                         np.reshape(log_alpha, (rows, H, dk)), np.reshape(d_o, (rows, H, dv)),
                         np.arange(B, dtype=np.int64) * T, np.full(B, T, dtype=np.int64),
                         initial_state, d_final_state, n_threads, lib)
    shapes = {"dq": (B, T, H, dk), "dk": (B, T, H, dk), "dv": (B, T, H, dv), "dbeta": (B, T, H),
              "dlog_alpha": (B, T, H, dk)}
    return {n: (x.reshape(shapes[n]) if n in shapes else x) for n, x in out.items()}


def varlen_backward(q, k, v, beta, log_alpha, d_o, cu_seqlens, initial_state=None,
                    d_final_state=None, n_threads: int = 0, lib=None):
    """``backward`` for a packed batch (layouts as ``varlen_prefill``; d_o
    [T_total, H, dv]; initial_state and d_final_state [N, H, dk, dv]).
    Returns the dict of ``backward``, token gradients [T_total, H, *]."""
    q = np.asarray(q)
    if q.ndim == 4:
        q, k, v, beta, log_alpha, d_o = (np.asarray(x)[0] for x in (q, k, v, beta, log_alpha, d_o))
    cu = np.asarray(cu_seqlens, dtype=np.int64)
    if cu.ndim != 1 or cu.shape[0] < 1 or cu[0] != 0 or np.any(np.diff(cu) < 0) \
            or cu[-1] != q.shape[0]:
        raise ValueError("cu_seqlens must start at 0, be non-decreasing and end at T_total")
    return _backward_rows(q, k, v, beta, log_alpha, d_o, cu[:-1], np.diff(cu), initial_state,
                          d_final_state, n_threads, lib)


def varlen_prefill(q, k, v, beta, log_alpha, cu_seqlens, initial_state=None,
                   n_threads: int = 0, lib=None, with_magnitude: bool = False):
    """Packed batch: q, k, log_alpha [T_total, H, dk] (a leading 1 is allowed);
    sequence n owns rows cu_seqlens[n] .. cu_seqlens[n+1]-1.

    Returns (o [T_total, H, dv], final_state [N, H, dk, dv]), float64.
    """
    q = np.asarray(q)
    if q.ndim == 4:
        q, k, v, beta, log_alpha = (np.asarray(x)[0] for x in (q, k, v, beta, log_alpha))
    cu = np.asarray(cu_seqlens, dtype=np.int64)
    if cu.ndim != 1 or cu.shape[0] < 1 or cu[0] != 0 or np.any(np.diff(cu) < 0) \
            or cu[-1] != q.shape[0]:
        raise ValueError("cu_seqlens must start at 0, be non-decreasing and end at T_total")
    return run_rows(q, k, v, beta, log_alpha, cu[:-1], np.diff(cu), 1,
                    initial_state, n_threads, lib, with_magnitude)


def decode_chain(q, k, v, beta, log_alpha, state, n_threads: int = 0, lib=None):
    """A chain of single-token steps: q, k, log_alpha [steps, N, H, dk];
    v [steps, N, H, dv]; beta [steps, N, H]; state [N, H, dk, dv] before step 0.

    Returns (o [steps, N, H, dv] -- the read-out of every step,
    final_state [N, H, dk, dv]), float64.
    """
    q = np.asarray(q)
    steps, N, H, dk = q.shape
    dv = np.asarray(v).shape[-1]
    row0 = np.arange(N, dtype=np.int64)
    length = np.full(N, steps, dtype=np.int64)
    o, s = run_rows(np.reshape(q, (steps * N, H, dk)), np.reshape(k, (steps * N, H, dk)),
                    np.reshape(v, (steps * N, H, dv)), np.reshape(beta, (steps * N, H)),
                    np.reshape(log_alpha, (steps * N, H, dk)), row0, length, N,
                    state, n_threads, lib)
    return o.reshape(steps, N, H, dv), s


def prepare(q_raw, k_raw, b_raw, a_raw, round_bf16: bool = True, lib=None):
    """Inputs from raw projections (see ``kda_oracle_prepare``): unit q and k
    per (token, head), rounded to bf16 when ``round_bf16``; beta =
    sigmoid(b_raw); log_alpha = -softplus(a_raw).  q_raw, k_raw, a_raw
    [..., H, dk]; b_raw [..., H].  Returns float32 (q, k, beta, log_alpha)."""
    lib = lib or load()
    q_raw = _f32(q_raw, "q_raw"); k_raw = _f32(k_raw, "k_raw")
    b_raw = _f32(b_raw, "b_raw"); a_raw = _f32(a_raw, "a_raw")
    H, dk = q_raw.shape[-2:]
    if k_raw.shape != q_raw.shape or a_raw.shape != q_raw.shape or b_raw.shape != q_raw.shape[:-1]:
        raise ValueError("q_raw, k_raw, a_raw must share [..., H, dk] and b_raw be [..., H]")
    rows = int(np.prod(q_raw.shape[:-2], dtype=np.int64))
    q, k = np.empty_like(q_raw), np.empty_like(k_raw)
    beta, la = np.empty_like(b_raw), np.empty_like(a_raw)
    rc = lib.kda_oracle_prepare(rows, H, dk, _ptr(q_raw, ctypes.c_float), _ptr(k_raw, ctypes.c_float),
                                _ptr(b_raw, ctypes.c_float), _ptr(a_raw, ctypes.c_float),
                                int(bool(round_bf16)), _ptr(q, ctypes.c_float), _ptr(k, ctypes.c_float),
                                _ptr(beta, ctypes.c_float), _ptr(la, ctypes.c_float))
    if rc != 0:
        raise RuntimeError(f"kda_oracle_prepare failed with code {rc}")
    return q, k, beta, la


def max_threads(n_threads: int = 0) -> int:
    return int(load().kda_oracle_max_threads(int(n_threads)))
