"""Cross-checks between the GPU entry points (each is also checked against
the oracle elsewhere): resuming from a stored state, decode == prefill, and
equivariance under a permutation of the value columns."""
import numpy as np
import pytest

import gated_delta_rule_113_amd as kda
import kda_inputs as ki
from kda_gpu import device, rel_err_states, rel_err_vectors, upload

pytestmark = pytest.mark.gpu


def test_resume_from_prefill_cache():
    """Prefill of T1 + T2 tokens == prefill of T1, then of T2 from the stored
    state (the prefill-cache resume)."""
    torch = __import__("torch")
    dev = device()
    inp = ki.dense_prefill(20, B=2, T=500, H=3, gated=True, initial_state=True)
    t = upload(inp, dev)
    o, S = kda.kda_prefill(t["q"], t["k"], t["v"], t["beta"], t["log_alpha"], t["initial_state"])
    for cut in (1, 64, 190, 499):
        sl = lambda x, a, b: x[:, a:b].contiguous()
        o1, S1 = kda.kda_prefill(*(sl(t[n], 0, cut) for n in ("q", "k", "v", "beta", "log_alpha")),
                                 t["initial_state"])
        o2, S2 = kda.kda_prefill(*(sl(t[n], cut, 500) for n in ("q", "k", "v", "beta", "log_alpha")),
                                 S1)
        torch.cuda.synchronize()
        oc = torch.cat([o1, o2], dim=1).cpu().numpy()
        assert rel_err_vectors(oc, o.cpu().numpy()) < 1e-4, cut
        assert rel_err_states(S2.cpu().numpy(), S.cpu().numpy()) < 1e-4, cut


def test_decode_chain_equals_prefill():
    """Feeding a sequence token by token through the decode step gives the
    prefill's outputs and final state."""
    torch = __import__("torch")
    dev = device()
    inp = ki.dense_prefill(21, B=2, T=70, H=2, gated=True, initial_state=True)
    t = upload(inp, dev)
    o, S = kda.kda_prefill(t["q"], t["k"], t["v"], t["beta"], t["log_alpha"], t["initial_state"])
    st = t["initial_state"].clone()
    outs = []
    for s in range(70):
        outs.append(kda.kda_decode_step(*(t[n][:, s].contiguous() for n in
                                          ("q", "k", "v", "beta", "log_alpha")), st))
    torch.cuda.synchronize()
    od = torch.stack(outs, dim=1).cpu().numpy()
    assert rel_err_vectors(od, o.cpu().numpy()) < 1e-4
    assert rel_err_states(st.cpu().numpy(), S.cpu().numpy()) < 1e-4


def test_value_column_permutation_equivariance():
    """Columns of the state are independent: permuting the value columns (v and
    the initial state's d_v axis) permutes the columns of o and of the final
    state and changes nothing else.  Checked for the chunked prefill (columns
    spread over waves and lanes), with segments, and for the decode step."""
    torch = __import__("torch")
    dev = device()
    perm = torch.from_numpy(np.random.default_rng(26).permutation(128)).to(dev)
    inp = ki.dense_prefill(26, B=1, T=300, H=2, gated=True, initial_state=True)
    t = upload(inp, dev)
    args = lambda vv: (t["q"], t["k"], vv, t["beta"], t["log_alpha"])
    for seg in (0, 64):
        kda.kda_set_prefill_segment(seg)
        try:
            o, S = kda.kda_prefill(*args(t["v"]), t["initial_state"])
            op, Sp = kda.kda_prefill(*args(t["v"][..., perm].contiguous()),
                                     t["initial_state"][..., perm].contiguous())
        finally:
            kda.kda_set_prefill_segment(0)
        torch.cuda.synchronize()
        assert rel_err_vectors(op.cpu().numpy(), o[..., perm].cpu().numpy()) < 1e-5, seg
        assert rel_err_states(Sp.cpu().numpy(), S[..., perm].cpu().numpy()) < 1e-5, seg
    d = upload(ki.decode_steps(26, steps=1, N=3, H=2), dev)
    st = d["initial_state"].clone()
    stp = d["initial_state"][..., perm].contiguous()
    o1 = kda.kda_decode_step(d["q"][0], d["k"][0], d["v"][0], d["beta"][0], d["log_alpha"][0], st)
    o2 = kda.kda_decode_step(d["q"][0], d["k"][0], d["v"][0][..., perm].contiguous(), d["beta"][0],
                             d["log_alpha"][0], stp)
    torch.cuda.synchronize()
    assert rel_err_vectors(o2.cpu().numpy(), o1[..., perm].cpu().numpy()) < 1e-5
    assert rel_err_states(stp.cpu().numpy(), st[..., perm].cpu().numpy()) < 1e-5
