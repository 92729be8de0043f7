"""Helpers for the GPU parity tests: upload seeded inputs, run the oracle on
the same bits, and measure the error the way the tolerance is stated.

Error metric (max relative error 2e-3 on outputs and final states, read per
vector / per matrix): for each output vector o_t of one (sequence, head,
token) the error is ||o_t - o_ref||_inf / ||o_ref||_inf; for each final state
of one (sequence, head) it is max|S - S_ref| / max|S_ref|.  The reported
error is the maximum over all of them.

A reference vector whose largest entry is below FLOOR = 1e-30 (for instance
the read-out right after a log-decay of -200 with nothing written) lies below
what an fp32 state can resolve; it is compared absolutely, |o - o_ref| <= FLOOR.

Cancellation.  The read-out o_t = S_t^T q_t is a sum of d_k = 128 terms; an
fp32 evaluation can be off by up to about d_k * 2^-24 times the magnitude of
those terms, m_t = |S_t|^T |q_t|, whatever the order of summation.  When the
terms cancel (e.g. the first token from a zero state gives o = beta (k.q) v,
and k.q can be 1e-6 of sum |k_i q_i|), o_t is far below m_t and no fp32
evaluation resolves it relative to its own norm.  Where the oracle supplies
m_t, the per-vector measure divides by max(||o_ref||_inf, ||m_t||_inf *
d_k 2^-24 / TOL): the tolerance then never asks for more than fp32 rounding of
the terms allows, and is unchanged for every vector whose terms do not cancel.
"""
from __future__ import annotations

import numpy as np

TOL = 2e-3
FLOOR = 1e-30
FP32_SUM_ERR = 128 * 2.0 ** -24   # relative rounding bound of a 128-term fp32 sum


def torch_mod():
    import torch
    return torch


def device():
    torch = torch_mod()
    if not torch.cuda.is_available():
        raise RuntimeError("these tests need a GPU")
    return torch.device("cuda", 0)


def to_dev(x, dtype_name, dev):
    """Upload a host array: uint16 bf16 bits -> torch.bfloat16, float32 as is."""
    torch = torch_mod()
    if dtype_name == "bf16" and x.dtype == np.uint16:
        return torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).view(torch.bfloat16).to(dev)
    return torch.from_numpy(np.ascontiguousarray(x)).to(dev)


def upload(inp, dev):
    """Device tensors (q, k, v, beta, log_alpha, initial_state, cu_seqlens)."""
    d = inp.dtype
    out = dict(q=to_dev(inp.q, d, dev), k=to_dev(inp.k, d, dev), v=to_dev(inp.v, d, dev),
               beta=to_dev(inp.beta, d, dev), log_alpha=to_dev(inp.log_alpha, "f32", dev))
    out["initial_state"] = None if inp.initial_state is None else to_dev(inp.initial_state, "f32", dev)
    out["cu_seqlens"] = None if inp.cu_seqlens is None else to_dev(inp.cu_seqlens, "i32", dev)
    return out


def rel_err_vectors(got, ref, mag=None):
    """Max over vectors (last axis) of ||got - ref||_inf / ||ref||_inf; with the
    oracle's read-out magnitudes ``mag`` the denominator is at least
    ||mag||_inf * FP32_SUM_ERR / TOL (see the module docstring)."""
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    assert got.shape == ref.shape, (got.shape, ref.shape)
    if got.size == 0:
        return 0.0
    assert np.all(np.isfinite(got)), "non-finite output"
    num = np.max(np.abs(got - ref), axis=-1)
    den = np.max(np.abs(ref), axis=-1)
    if mag is not None:
        den = np.maximum(den, np.max(np.abs(np.asarray(mag, np.float64)), axis=-1) * (FP32_SUM_ERR / TOL))
    tiny = den < FLOOR
    if np.any(tiny):
        assert np.all(num[tiny] <= FLOOR), "output far from a reference below the fp32 floor"
    if np.all(tiny):
        return 0.0
    return float(np.max(num[~tiny] / den[~tiny]))


def rel_err_states(got, ref):
    """Max over [d_k, d_v] state matrices of max|got - ref| / max|ref|."""
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    assert got.shape == ref.shape, (got.shape, ref.shape)
    g = got.reshape(-1, got.shape[-2] * got.shape[-1])
    r = ref.reshape(g.shape)
    assert np.all(np.isfinite(g)), "non-finite state"
    num = np.max(np.abs(g - r), axis=-1)
    den = np.max(np.abs(r), axis=-1)
    tiny = den < FLOOR
    if np.any(tiny):
        assert np.all(num[tiny] <= FLOOR), "state far from a reference below the fp32 floor"
    if np.all(tiny):
        return 0.0
    return float(np.max(num[~tiny] / den[~tiny]))


def check(name, o_err, s_err, tol=TOL):
    print(f"{name}: max rel err o={o_err:.3e} state={s_err:.3e} (tol {tol:g})", flush=True)
    assert o_err <= tol, f"{name}: output error {o_err:.3e} > {tol}"
    assert s_err <= tol, f"{name}: state error {s_err:.3e} > {tol}"


class GroupCheck:
    """Accumulates the error metric over groups of heads or sequences that the
    oracle recomputes one after another (to keep host memory bounded), and
    the oracle's wall time, then checks the maxima against the tolerance."""

    def __init__(self, name):
        self.name = name
        self.o_err = 0.0
        self.s_err = 0.0
        self.oracle_s = 0.0
        self.units = 0

    def timed(self, fn, *args, **kw):
        import time
        t0 = time.time()
        out = fn(*args, **kw)
        self.oracle_s += time.time() - t0
        return out

    def add(self, o_err, s_err, units):
        self.o_err = max(self.o_err, o_err)
        self.s_err = max(self.s_err, s_err)
        self.units += units

    def finish(self, tol=TOL):
        import oracle
        print(f"{self.name}: oracle recomputed {self.units} (sequence, head) units in "
              f"{self.oracle_s:.1f}s wall on {oracle.max_threads()} threads", flush=True)
        check(self.name, self.o_err, self.s_err, tol)
