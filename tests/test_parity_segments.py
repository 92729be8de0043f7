"""Segmented (sequence-parallel) bf16 prefill on the GPU vs the fp64 oracle.

Long sequences are cut into segments whose affine state maps are composed on
the device; these tests force short segments so that small problems, which
the oracle finishes quickly, take that path with many segments, ragged last
segments and every pass of it."""
import numpy as np
import pytest

import gated_delta_rule_113_amd as kda
import kda_inputs as ki
import oracle
from kda_gpu import check, device, rel_err_states, rel_err_vectors, upload

pytestmark = pytest.mark.gpu


@pytest.fixture
def segment():
    """Set a forced segment length for one test, then restore automatic."""
    def set_(tokens):
        kda.kda_set_prefill_segment(tokens)
    yield set_
    kda.kda_set_prefill_segment(0)


def _dense(inp, dev, **kw):
    torch = __import__("torch")
    t = upload(inp, dev)
    o, S = kda.kda_prefill(t["q"], t["k"], t["v"], t["beta"], t["log_alpha"], t["initial_state"], **kw)
    torch.cuda.synchronize()
    return o.cpu().numpy(), S.cpu().numpy()


def _varlen(inp, dev, **kw):
    torch = __import__("torch")
    t = upload(inp, dev)
    o, S = kda.kda_varlen_prefill(t["q"], t["k"], t["v"], t["beta"], t["log_alpha"],
                                  t["cu_seqlens"], t["initial_state"], **kw)
    torch.cuda.synchronize()
    return o.cpu().numpy(), S.cpu().numpy()


@pytest.mark.parametrize("seg,T", [(64, 500), (128, 500), (192, 383), (256, 257), (128, 128)])
def test_dense_segmented(segment, seg, T):
    """Two sequences, three heads, gated channel mix, resumed states; the
    segment length does not divide T (except the last case, one segment)."""
    inp = ki.dense_prefill(40, B=2, T=T, H=3, gated=True, initial_state=True)
    segment(seg)
    o, S = _dense(inp, device())
    o_ref, S_ref = oracle.prefill(*inp.widened(), inp.initial_state)
    check(f"dense segmented seg={seg} T={T}", rel_err_vectors(o, o_ref), rel_err_states(S, S_ref))


def test_dense_automatic_segments():
    """Automatic segment lengths for dense input: at B=2, H=8, T=4096 on 256
    compute units each sequence is cut into four segments of 1024 tokens; the
    first runs with outputs in pass 1, pass 3 reuses the T and P of the next
    two and forms those of the last; resumed (non-zero) initial states."""
    inp = ki.dense_prefill(42, B=2, T=4096, H=8, gated=True, initial_state=True)
    o, S = _dense(inp, device())
    o_ref, S_ref = oracle.prefill(*inp.widened(), inp.initial_state)
    check("dense automatic segments", rel_err_vectors(o, o_ref), rel_err_states(S, S_ref))


def _segments_workspace(B, T, H, packed_n=None):
    """A caller workspace of exactly the KDA_PLAN_SEGMENTS size (segments
    without the T/P images), which the call then takes."""
    torch = __import__("torch")
    if packed_n is None:
        n = kda.prefill_workspace_size(B, T, H, torch.bfloat16, kda.KDA_PLAN_SEGMENTS)
        full = kda.prefill_workspace_size(B, T, H, torch.bfloat16, kda.KDA_PLAN_FULL)
    else:
        n = kda.varlen_prefill_workspace_size(packed_n, T, H, torch.bfloat16, kda.KDA_PLAN_SEGMENTS)
        full = kda.varlen_prefill_workspace_size(packed_n, T, H, torch.bfloat16, kda.KDA_PLAN_FULL)
    assert 0 < n < full
    return torch.empty(n, dtype=torch.uint8, device=device())


def test_dense_automatic_without_tp_workspace():
    """Without the T/P images (a workspace of the KDA_PLAN_SEGMENTS size) the
    automatic lengths at B=2, H=8, T=4096 are 896 (first segment, with outputs
    in pass 1), three of 1024 and 128, and every pass-3 segment forms its own
    T and P."""
    inp = ki.dense_prefill(43, B=2, T=4096, H=8, gated=True, initial_state=True)
    o, S = _dense(inp, device(), workspace=_segments_workspace(2, 4096, 8))
    o_ref, S_ref = oracle.prefill(*inp.widened(), inp.initial_state)
    check("dense automatic segments, no T/P reuse", rel_err_vectors(o, o_ref), rel_err_states(S, S_ref))


def test_dense_forced_segments_without_tp_workspace(segment):
    inp = ki.dense_prefill(44, B=2, T=500, H=3, gated=True, initial_state=True)
    segment(64)
    o, S = _dense(inp, device(), workspace=_segments_workspace(2, 500, 3))
    o_ref, S_ref = oracle.prefill(*inp.widened(), inp.initial_state)
    check("dense segmented seg=64, no T/P reuse", rel_err_vectors(o, o_ref), rel_err_states(S, S_ref))


def test_dense_segmented_zero_initial_state(segment):
    inp = ki.dense_prefill(41, B=1, T=700, H=2, gated=True)
    segment(64)
    o, S = _dense(inp, device())
    o_ref, S_ref = oracle.prefill(*inp.widened(), None)
    check("dense segmented, zero S0", rel_err_vectors(o, o_ref), rel_err_states(S, S_ref))


def test_dense_segmented_aliased_state(segment):
    """final_state aliasing initial_state is safe on the segmented path."""
    torch = __import__("torch")
    dev = device()
    inp = ki.dense_prefill(42, B=2, T=450, H=2, gated=True, initial_state=True)
    o_ref, S_ref = oracle.prefill(*inp.widened(), inp.initial_state)
    segment(128)
    t = upload(inp, dev)
    st = t["initial_state"].clone()
    o, S = kda.kda_prefill(t["q"], t["k"], t["v"], t["beta"], t["log_alpha"], st, final_state=st)
    torch.cuda.synchronize()
    check("segmented aliased", rel_err_vectors(o.cpu().numpy(), o_ref),
          rel_err_states(S.cpu().numpy(), S_ref))


@pytest.mark.parametrize("tp", [True, False])
def test_varlen_segmented(segment, tp):
    """Packed sequences of lengths 0, 1, 63, 64, 65, 300, 0, 129, 520 with
    segments of 128 tokens: some sequences have one segment, some five; with
    and without the T/P reuse."""
    inp = ki.varlen_prefill(43, [0, 1, 63, 64, 65, 300, 0, 129, 520], H=3)
    segment(128)
    ws = None if tp else _segments_workspace(None, int(inp.cu_seqlens[-1]), 3, packed_n=9)
    o, S = _varlen(inp, device(), workspace=ws)
    q, k, v, b, la = inp.widened()
    o_ref, S_ref = oracle.varlen_prefill(q, k, v, b, la, inp.cu_seqlens, inp.initial_state)
    check("varlen segmented", rel_err_vectors(o[0], o_ref), rel_err_states(S, S_ref))
    assert np.array_equal(S[0], inp.initial_state[0])
    assert np.array_equal(S[6], inp.initial_state[6])


def test_segmented_equals_unsegmented(segment):
    """The same problem with and without segmentation agrees to rounding."""
    inp = ki.dense_prefill(44, B=1, T=1000, H=4, gated=True, initial_state=True)
    dev = device()
    segment(0)
    o1, S1 = _dense(inp, dev)
    segment(192)
    o2, S2 = _dense(inp, dev)
    assert rel_err_vectors(o2, o1) < 1e-4
    assert rel_err_states(S2, S1) < 1e-4


def test_segmented_extreme_gates(segment):
    """Segment maps under channels that forget almost completely in one token
    and channels that never forget."""
    inp = ki.dense_prefill(45, B=1, T=400, H=2, gated=True, initial_state=True)
    r = np.random.default_rng(45)
    la = inp.log_alpha
    la[0, r.integers(0, 400, 40), 0, :] = -200.0
    la[0, :, 1, :5] = 0.0
    la[0, 100:140, 1, 64:] = -60.0
    segment(64)
    o, S = _dense(inp, device())
    o_ref, S_ref = oracle.prefill(*inp.widened(), inp.initial_state)
    check("segmented extreme gates", rel_err_vectors(o, o_ref), rel_err_states(S, S_ref))
