"""The largest head count the library accepts, on the GPU.

H = 65,536 is the limit because the kernels address a chunk's inputs with
32-bit byte offsets from the chunk's first row: one 64-token chunk of fp32
gates then spans 2 GB.  At that head count: the chunked prefill (a full chunk
and a ragged one), the short-sequence path, a decode step and the backward
pass, each from
random initial states, with sampled heads (the first, the last and two in
between) against the oracle.  Inputs are drawn on the GPU (seeded); the
sampled heads are copied back exactly (bf16 widens exactly to fp32).
"""
import numpy as np
import pytest

import gated_delta_rule_113_amd as kda
import oracle
from kda_gpu import check, device, rel_err_states, rel_err_vectors

pytestmark = pytest.mark.gpu

H = 65536
HEADS = [0, 1, 40961, H - 1]


def _torch():
    import torch
    return torch


def _draw(rows_shape, seed):
    """q, k (unit vectors), v, beta, log_alpha and an initial state on the GPU."""
    torch = _torch()
    dev = device()
    g = torch.Generator(device=dev).manual_seed(seed)
    unit = lambda x: x / x.norm(dim=-1, keepdim=True)
    q = unit(torch.randn(*rows_shape, H, 128, device=dev, generator=g)).to(torch.bfloat16)
    k = unit(torch.randn(*rows_shape, H, 128, device=dev, generator=g)).to(torch.bfloat16)
    v = torch.randn(*rows_shape, H, 128, device=dev, generator=g).to(torch.bfloat16)
    beta = torch.sigmoid(torch.randn(*rows_shape, H, device=dev, generator=g)).to(torch.bfloat16)
    la = -torch.nn.functional.softplus(torch.randn(*rows_shape, H, 128, device=dev, generator=g))
    return q, k, v, beta, la


def _host(x, head_axis):
    torch = _torch()
    idx = torch.tensor(HEADS, device=x.device)
    return x.index_select(head_axis, idx).float().cpu().numpy()


@pytest.mark.parametrize("T", [70, 9])
def test_prefill_max_heads(T):
    """T = 70 runs the chunked kernel (a full 64-token chunk, then 6 tokens);
    T = 9 the short-sequence kernel."""
    torch = _torch()
    dev = device()
    q, k, v, beta, la = _draw((1, T), seed=T)
    g = torch.Generator(device=dev).manual_seed(1000 + T)
    s0 = torch.randn(1, H, 128, 128, device=dev, generator=g) * 0.02
    o, S = kda.kda_prefill(q, k, v, beta, la, s0)
    torch.cuda.synchronize()
    o_h, S_h = _host(o, 2), _host(S, 1)
    o_ref, S_ref = oracle.prefill(_host(q, 2), _host(k, 2), _host(v, 2), _host(beta, 2),
                                  _host(la, 2), _host(s0, 1))
    check(f"prefill H={H} T={T}, sampled heads", rel_err_vectors(o_h, o_ref),
          rel_err_states(S_h, S_ref))


def test_decode_max_heads():
    torch = _torch()
    dev = device()
    q, k, v, beta, la = _draw((1,), seed=3)
    g = torch.Generator(device=dev).manual_seed(1003)
    state = torch.randn(1, H, 128, 128, device=dev, generator=g) * 0.02
    s0_h = _host(state, 1)
    o = kda.kda_decode_step(q, k, v, beta, la, state)
    torch.cuda.synchronize()
    o_ref, S_ref = oracle.decode_chain(_host(q, 1)[None], _host(k, 1)[None], _host(v, 1)[None],
                                       _host(beta, 1)[None], _host(la, 1)[None], s0_h)
    check(f"decode H={H}, sampled heads", rel_err_vectors(_host(o, 1), o_ref[0]),
          rel_err_states(_host(state, 1), S_ref))


def test_backward_max_heads():
    """The backward pass at H = 65,536 (9 tokens: a full checkpoint block and
    one more), from random states, all gradients of the sampled heads against
    the oracle.  The loss gradients are drawn on the GPU as well."""
    torch = _torch()
    dev = device()
    T = 9
    q, k, v, beta, la = _draw((1, T), seed=20)
    g = torch.Generator(device=dev).manual_seed(1020)
    s0 = torch.randn(1, H, 128, 128, device=dev, generator=g) * 0.02
    d_o = torch.randn(1, T, H, 128, device=dev, generator=g)
    d_s = torch.randn(1, H, 128, 128, device=dev, generator=g)
    out = kda.kda_backward(q, k, v, beta, la, d_o, s0, d_s)
    torch.cuda.synchronize()
    ref = oracle.backward(_host(q, 2), _host(k, 2), _host(v, 2), _host(beta, 2), _host(la, 2),
                          _host(d_o, 2), _host(s0, 1), _host(d_s, 1))
    errs = {n: rel_err_vectors(_host(out[n], 2), ref[n]) for n in ("dq", "dk", "dv", "dlog_alpha")}
    errs["dbeta"] = rel_err_vectors(_host(out["dbeta"], 2)[0].T, ref["dbeta"][0].T)
    errs["dinitial_state"] = rel_err_states(_host(out["dinitial_state"], 1), ref["dinitial_state"])
    print("backward H=65536 T=9, sampled heads: " + " ".join(f"{n}={e:.2e}" for n, e in errs.items()),
          flush=True)
    for n, e in errs.items():
        assert e <= 2e-3, (n, e)
