"""Dense prefill on the GPU vs the fp64 oracle."""
import numpy as np
import pytest

import gated_delta_rule_113_amd as kda
import kda_inputs as ki
import oracle
from kda_gpu import GroupCheck, check, device, rel_err_states, rel_err_vectors, upload

pytestmark = pytest.mark.gpu


def _run(inp, dev, **kw):
    torch = __import__("torch")
    t = upload(inp, dev)
    o, S = kda.kda_prefill(t["q"], t["k"], t["v"], t["beta"], t["log_alpha"],
                           t["initial_state"], **kw)
    torch.cuda.synchronize()
    return o.cpu().numpy(), S.cpu().numpy()


def _oracle(inp):
    q, k, v, b, la = inp.widened()
    return oracle.prefill(q, k, v, b, la, inp.initial_state)


def test_single_sequence_fp32():
    """B=1, H=1, T=256, everything fp32, zero initial state."""
    inp = ki.workload_single()
    o, S = _run(inp, device())
    o_ref, S_ref = _oracle(inp)
    check("single fp32", rel_err_vectors(o, o_ref), rel_err_states(S, S_ref))


@pytest.mark.parametrize("T", [1, 2, 63, 64, 65, 127, 128, 129, 200])
def test_ragged_lengths_with_initial_state(T):
    """Lengths around the 64-token chunk boundary, bf16 inputs, gated channel
    mix, non-zero initial state, two sequences of three heads."""
    inp = ki.dense_prefill(5, B=2, T=T, H=3, gated=True, initial_state=True)
    o, S = _run(inp, device())
    o_ref, S_ref = _oracle(inp)
    check(f"ragged T={T}", rel_err_vectors(o, o_ref), rel_err_states(S, S_ref))


def test_chunked_reduced():
    """The chunked-prefill workload at H=4, T=4096 (64 chunks), checked in full."""
    inp = ki.workload_chunked(T=4096, H=4)
    o, S = _run(inp, device())
    o_ref, S_ref = _oracle(inp)
    check("chunked H=4 T=4096", rel_err_vectors(o, o_ref), rel_err_states(S, S_ref))


def test_chunked_full_size_every_head():
    """The full chunked-prefill workload (H=32, T=32768) in the launch
    configuration the benchmark times; the oracle recomputes every head in
    full (all outputs and final states), 8 heads at a time."""
    inp = ki.workload_chunked()
    o, S = _run(inp, device())
    assert np.all(np.isfinite(o)) and np.all(np.isfinite(S))
    H = inp.q.shape[2]
    gc = GroupCheck(f"chunked full, all {H} heads")
    for h0 in range(0, H, 8):
        hs = slice(h0, h0 + 8)
        w = [ki.bf16_to_f32(np.ascontiguousarray(x[:, :, hs])) for x in (inp.q, inp.k, inp.v, inp.beta)]
        la = np.ascontiguousarray(inp.log_alpha[:, :, hs])
        o_ref, S_ref = gc.timed(oracle.prefill, *w, la, None)
        gc.add(rel_err_vectors(o[:, :, hs], o_ref), rel_err_states(S[:, hs], S_ref), 8)
    assert gc.units == H
    gc.finish()


def test_empty_sequence_returns_initial_state():
    torch = __import__("torch")
    dev = device()
    inp = ki.dense_prefill(6, B=2, T=0, H=2, initial_state=True)
    t = upload(inp, dev)
    o, S = kda.kda_prefill(t["q"], t["k"], t["v"], t["beta"], t["log_alpha"], t["initial_state"])
    torch.cuda.synchronize()
    assert o.shape == (2, 0, 2, 128)
    assert torch.equal(S, t["initial_state"])
    o, S = kda.kda_prefill(t["q"], t["k"], t["v"], t["beta"], t["log_alpha"], None)
    torch.cuda.synchronize()
    assert torch.count_nonzero(S) == 0


def test_final_state_may_alias_initial_state():
    torch = __import__("torch")
    dev = device()
    inp = ki.dense_prefill(7, B=2, T=150, H=2, gated=True, initial_state=True)
    o_ref, S_ref = _oracle(inp)
    t = upload(inp, dev)
    st = t["initial_state"].clone()
    o, S = kda.kda_prefill(t["q"], t["k"], t["v"], t["beta"], t["log_alpha"], st, final_state=st)
    torch.cuda.synchronize()
    assert S.data_ptr() == st.data_ptr()
    check("aliased state", rel_err_vectors(o.cpu().numpy(), o_ref),
          rel_err_states(S.cpu().numpy(), S_ref))


def test_extreme_gates():
    """Channels that forget almost completely in one token (log_alpha = -200),
    channels that never forget (log_alpha = 0), beta at 0 and 1."""
    inp = ki.dense_prefill(8, B=1, T=300, H=2, gated=True, initial_state=True)
    r = np.random.default_rng(8)
    la = inp.log_alpha
    la[0, r.integers(0, 300, 40), 0, :] = -200.0
    la[0, :, 1, :5] = 0.0
    la[0, 100:140, 1, 64:] = -60.0
    bb = ki.bf16_to_f32(inp.beta)
    bb[0, ::7, 0] = 0.0
    bb[0, ::5, 1] = 1.0
    inp.beta = ki.bf16_bits(bb)
    o, S = _run(inp, device())
    o_ref, S_ref = _oracle(inp)
    check("extreme gates", rel_err_vectors(o, o_ref), rel_err_states(S, S_ref))


def test_deterministic():
    """Two runs give identical bits (no atomics, no races)."""
    inp = ki.dense_prefill(9, B=1, T=333, H=4, gated=True, initial_state=True)
    dev = device()
    o1, S1 = _run(inp, dev)
    o2, S2 = _run(inp, dev)
    assert np.array_equal(o1, o2) and np.array_equal(S1, S2)


def test_many_heads_segmented():
    """96 heads (beyond the workloads' 32, not a power of two): two dense
    sequences of 300 tokens cut into 128-token segments, so that every launch
    maps its workgroups to (segment, head) pairs over 96 heads."""
    inp = ki.dense_prefill(10, B=2, T=300, H=96, gated=True, initial_state=True)
    kda.kda_set_prefill_segment(128)
    try:
        o, S = _run(inp, device())
    finally:
        kda.kda_set_prefill_segment(0)
    o_ref, S_ref = _oracle(inp)
    check("96 heads, segmented", rel_err_vectors(o, o_ref), rel_err_states(S, S_ref))
