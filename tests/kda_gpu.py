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
"""
from __future__ import annotations

import numpy as np

TOL = 2e-3
FLOOR = 1e-30


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


def rel_err_vectors(got, ref):
    """Max over vectors (last axis) of ||got - ref||_inf / ||ref||_inf."""
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    assert got.shape == ref.shape, (got.shape, ref.shape)
    if got.size == 0:
        return 0.0
    assert np.all(np.isfinite(got)), "non-finite output"
    num = np.max(np.abs(got - ref), axis=-1)
    den = np.max(np.abs(ref), axis=-1)
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
