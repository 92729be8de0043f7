"""Decode step on the GPU vs the fp64 oracle (batched decode workload:
B sequences x H heads, consecutive single-token steps, bf16 q/k/v/beta, fp32
log_alpha and state, states starting from N(0, 0.02^2))."""
import numpy as np
import pytest

import gated_delta_rule_113_amd as kda
import kda_inputs as ki
import oracle
from kda_gpu import GroupCheck, check, device, rel_err_states, rel_err_vectors, upload

pytestmark = pytest.mark.gpu


def _run_chain(inp, dev):
    torch = __import__("torch")
    t = upload(inp, dev)
    state = t["initial_state"].clone()
    outs = []
    for s in range(inp.q.shape[0]):
        outs.append(kda.kda_decode_step(t["q"][s], t["k"][s], t["v"][s], t["beta"][s],
                                        t["log_alpha"][s], state))
    torch.cuda.synchronize()
    return torch.stack(outs).cpu().numpy(), state.cpu().numpy()


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_decode_small_every_step(dtype):
    inp = ki.decode_steps(1, steps=64, N=4, H=4, dtype=dtype)
    o, S = _run_chain(inp, device())
    q, k, v, b, la = inp.widened()
    o_ref, S_ref = oracle.decode_chain(q, k, v, b, la, inp.initial_state)
    check(f"decode small {dtype}", rel_err_vectors(o, o_ref), rel_err_states(S, S_ref))


def test_decode_full_size_every_head():
    """The full workload (64 sequences x 32 heads, 1024 steps) in the launch
    configuration the benchmark times: every head's output at every step and
    every final state are checked against the oracle, which recomputes the
    chain 8 sequences (256 heads) at a time."""
    inp = ki.workload_decode()
    steps, N, H = inp.q.shape[:3]
    o, S = _run_chain(inp, device())
    assert np.all(np.isfinite(o)) and np.all(np.isfinite(S))
    gc = GroupCheck(f"decode full, all {N * H} heads x {steps} steps")
    for n0 in range(0, N, 8):
        ns = slice(n0, n0 + 8)
        w = [ki.bf16_to_f32(np.ascontiguousarray(x[:, ns])) for x in (inp.q, inp.k, inp.v, inp.beta)]
        la = np.ascontiguousarray(inp.log_alpha[:, ns])
        o_ref, S_ref = gc.timed(oracle.decode_chain, *w, la, inp.initial_state[ns])
        gc.add(rel_err_vectors(o[:, ns], o_ref), rel_err_states(S[ns], S_ref), 8 * H)
    assert gc.units == N * H
    gc.finish()


def test_decode_streamed_state_every_head():
    """A batch whose states (136 sequences x 32 heads, 272 MiB) exceed the
    256 MB last-level cache, which the step streams with the nontemporal
    hint: two steps, every head's outputs and final state against the oracle."""
    inp = ki.decode_steps(7, steps=2, N=136, H=32)
    o, S = _run_chain(inp, device())
    assert np.all(np.isfinite(o)) and np.all(np.isfinite(S))
    q, k, v, b, la = inp.widened()
    o_ref, S_ref = oracle.decode_chain(q, k, v, b, la, inp.initial_state)
    check("decode streamed state, 136 x 32 heads", rel_err_vectors(o, o_ref), rel_err_states(S, S_ref))


def test_decode_in_place_and_zero_beta():
    """beta = 0 and log_alpha = 0 leave the state bit-for-bit unchanged; the
    output is then S^T q."""
    torch = __import__("torch")
    dev = device()
    inp = ki.decode_steps(1, steps=1, N=3, H=2)
    t = upload(inp, dev)
    state = t["initial_state"].clone()
    before = state.clone()
    o = kda.kda_decode_step(t["q"][0], t["k"][0], t["v"][0], torch.zeros_like(t["beta"][0]),
                            torch.zeros_like(t["log_alpha"][0]), state)
    torch.cuda.synchronize()
    assert torch.equal(state, before)
    q = t["q"][0].float().cpu().numpy().astype(np.float64)
    ref = np.einsum("nhij,nhi->nhj", before.cpu().numpy().astype(np.float64), q)
    assert rel_err_vectors(o.cpu().numpy(), ref) < 1e-5


def test_decode_many_heads():
    """96 heads for 5 sequences, 8 consecutive steps."""
    inp = ki.decode_steps(2, steps=8, N=5, H=96)
    o, S = _run_chain(inp, device())
    o_ref, S_ref = oracle.decode_chain(*inp.widened(), inp.initial_state)
    check("decode 96 heads", rel_err_vectors(o, o_ref), rel_err_states(S, S_ref))
