"""Backward pass on the GPU (kda_backward, kda_varlen_backward) vs the fp64
oracle's backward, which is pinned against finite differences of the forward
oracle.

Every gradient is compared with the error measure of the forward outputs: per
vector (one token and head: dq, dk, dv, d log alpha; one sequence and head
over its tokens: d beta) and per matrix (d initial state), max over all, at
most 2e-3.  bf16 inputs take the chunked form on the matrix cores (64-token chunks,
split-bf16 products with fp32 accumulation), fp32 inputs the token-by-token
chain rule in fp32; the measured errors are far below the tolerance.
"""
import numpy as np
import pytest

import gated_delta_rule_113_amd as kda
import kda_inputs as ki
import oracle
from kda_gpu import TOL, device, rel_err_states, rel_err_vectors, to_dev, upload

pytestmark = pytest.mark.gpu

TOKEN_GRADS = ("dq", "dk", "dv", "dlog_alpha")


def _compare(name, got, ref, tol=TOL):
    errs = {n: rel_err_vectors(got[n], ref[n]) for n in TOKEN_GRADS}
    # d beta: one value per (token, head); compared per head over the tokens
    errs["dbeta"] = rel_err_vectors(np.swapaxes(got["dbeta"], -1, -2),
                                    np.swapaxes(ref["dbeta"], -1, -2))
    errs["dinitial_state"] = rel_err_states(got["dinitial_state"], ref["dinitial_state"])
    print(f"{name}: " + " ".join(f"{n}={e:.2e}" for n, e in errs.items()) + f" (tol {tol:g})",
          flush=True)
    for n, e in errs.items():
        assert e <= tol, f"{name}: {n} error {e:.3e} > {tol}"


def _host(g):
    return {n: x.cpu().numpy() for n, x in g.items()}


def _dense(inp, d_o, d_s, dev):
    torch = __import__("torch")
    t = upload(inp, dev)
    g = kda.kda_backward(t["q"], t["k"], t["v"], t["beta"], t["log_alpha"], to_dev(d_o, "f32", dev),
                         t["initial_state"], None if d_s is None else to_dev(d_s, "f32", dev))
    torch.cuda.synchronize()
    return _host(g)


def test_backward_dense_bf16():
    """Two sequences of 150 tokens (two chunks of 64 and a ragged 22), three
    heads, the gated channel mix, resumed states, both loss gradients."""
    B, T, H = 2, 150, 3
    inp = ki.dense_prefill(40, B=B, T=T, H=H, gated=True, initial_state=True)
    d_o, d_s = ki.loss_gradients(40, (B, T, H, 128), B, H)
    got = _dense(inp, d_o, d_s, device())
    ref = oracle.backward(*inp.widened(), d_o, inp.initial_state, d_s)
    _compare("backward dense bf16", got, ref)


def test_backward_extreme_gates():
    """Tokens whose every channel forgets completely (log_alpha = -200), some
    of them inside a run of -20 on channels 20..39 (decays beyond 2^-96 over
    half a 16-token block, so the diagonal blocks take those channels
    pairwise), a run of -60 on half the channels of the other head, channels
    that never forget (log_alpha = 0), beta at 0 and 1 (a token after a -200
    one with beta = 0 enters from a vanishing state, so its d log alpha is of
    order e^-200); resumed states, both loss gradients."""
    inp = ki.dense_prefill(57, B=1, T=300, H=2, gated=True, initial_state=True)
    r = np.random.default_rng(57)
    la = inp.log_alpha
    la[0, r.integers(0, 300, 40), 0, :] = -200.0
    la[0, :, 1, :5] = 0.0
    la[0, 100:140, 1, 64:] = -60.0
    la[0, 150:230, 0, 20:40] = -20.0
    bb = ki.bf16_to_f32(inp.beta)
    bb[0, ::7, 0] = 0.0
    bb[0, ::5, 1] = 1.0
    inp.beta = ki.bf16_bits(bb)
    d_o, d_s = ki.loss_gradients(57, (1, 300, 2, 128), 1, 2)
    got = _dense(inp, d_o, d_s, device())
    ref = oracle.backward(*inp.widened(), d_o, inp.initial_state, d_s)
    _compare("backward extreme gates", got, ref)


def test_backward_fp32_inputs_no_states():
    """fp32 inputs, no initial state and no final-state gradient (zeros)."""
    inp = ki.workload_single(T=256)
    d_o, _ = ki.loss_gradients(41, (1, 256, 1, 128), 1, 1)
    got = _dense(inp, d_o, None, device())
    ref = oracle.backward(*inp.widened(), d_o)
    _compare("backward fp32", got, ref)


@pytest.mark.parametrize("T", [1, 7, 63, 64, 65])
def test_backward_short_sequences(T):
    """bf16: within one chunk, exactly one chunk, one token more."""
    inp = ki.dense_prefill(42 + T, B=3, T=T, H=2, gated=True, initial_state=True)
    d_o, d_s = ki.loss_gradients(42 + T, (3, T, 2, 128), 3, 2)
    got = _dense(inp, d_o, d_s, device())
    ref = oracle.backward(*inp.widened(), d_o, inp.initial_state, d_s)
    _compare(f"backward T={T}", got, ref)


@pytest.mark.parametrize("T", [1, 7, 8, 9, 70])
def test_backward_fp32_checkpoint_blocks(T):
    """fp32 inputs (the token-by-token path): fewer tokens than one
    checkpoint block of 8, exactly one, one more, and several with a ragged
    last block; resumed states and both loss gradients."""
    inp = ki.dense_prefill(60 + T, B=2, T=T, H=2, dtype="f32", gated=True, initial_state=True)
    d_o, d_s = ki.loss_gradients(60 + T, (2, T, 2, 128), 2, 2)
    got = _dense(inp, d_o, d_s, device())
    ref = oracle.backward(*inp.widened(), d_o, inp.initial_state, d_s)
    _compare(f"backward fp32 T={T}", got, ref)


def test_backward_no_tokens():
    """T = 0: the initial-state gradient is the final-state gradient, bit for
    bit (zeros when none is given)."""
    torch = __import__("torch")
    dev = device()
    H = 2
    z = torch.zeros((1, 0, H, 128), dtype=torch.bfloat16, device=dev)
    b = torch.zeros((1, 0, H), dtype=torch.bfloat16, device=dev)
    la = torch.zeros((1, 0, H, 128), dtype=torch.float32, device=dev)
    d_o = torch.zeros((1, 0, H, 128), dtype=torch.float32, device=dev)
    _, d_s = ki.loss_gradients(50, (1, 0, H, 128), 1, H)
    ds_dev = to_dev(d_s, "f32", dev)
    g = kda.kda_backward(z, z, z, b, la, d_o, None, ds_dev)
    g0 = kda.kda_backward(z, z, z, b, la, d_o)
    torch.cuda.synchronize()
    assert np.array_equal(g["dinitial_state"].cpu().numpy(), d_s)
    assert not g0["dinitial_state"].cpu().numpy().any()


def test_backward_varlen():
    """Packed sequences of 0, 1, 7, 8, 9, 70, 0 and 33 tokens (even ones
    resumed): per-sequence recurrences, empty ones pass the final-state
    gradient through unchanged."""
    torch = __import__("torch")
    dev = device()
    lengths = [0, 1, 7, 8, 9, 70, 0, 33]
    H = 2
    inp = ki.varlen_prefill(51, lengths, H=H)
    Tt = int(sum(lengths))
    d_o, d_s = ki.loss_gradients(51, (1, Tt, H, 128), len(lengths), H)
    t = upload(inp, dev)
    g = kda.kda_varlen_backward(t["q"], t["k"], t["v"], t["beta"], t["log_alpha"],
                                to_dev(d_o, "f32", dev), t["cu_seqlens"], t["initial_state"],
                                to_dev(d_s, "f32", dev))
    torch.cuda.synchronize()
    got = _host(g)
    ref = oracle.varlen_backward(*inp.widened(), d_o, inp.cu_seqlens, inp.initial_state, d_s)
    got = {n: (x[0] if n != "dinitial_state" else x) for n, x in got.items()}
    _compare("backward varlen", got, ref)
    assert np.array_equal(got["dinitial_state"][0], d_s[0])
    assert np.array_equal(got["dinitial_state"][6], d_s[6])


def test_backward_long_gated():
    """2048 tokens (32 chunks), four heads, gated mix: long-memory channels
    carry the gradient over the whole sequence, through 32 chunk steps of the
    state and gradient sweeps."""
    B, T, H = 1, 2048, 4
    inp = ki.dense_prefill(52, B=B, T=T, H=H, gated=True, initial_state=True)
    d_o, d_s = ki.loss_gradients(52, (B, T, H, 128), B, H)
    got = _dense(inp, d_o, d_s, device())
    ref = oracle.backward(*inp.widened(), d_o, inp.initial_state, d_s)
    _compare("backward T=2048", got, ref)


def test_backward_long_ragged():
    """Two sequences of 3500 tokens (54 full chunks and a ragged 44), two
    heads, resumed states."""
    B, T, H = 2, 3500, 2
    inp = ki.dense_prefill(56, B=B, T=T, H=H, gated=True, initial_state=True)
    d_o, d_s = ki.loss_gradients(56, (B, T, H, 128), B, H)
    got = _dense(inp, d_o, d_s, device())
    ref = oracle.backward(*inp.widened(), d_o, inp.initial_state, d_s)
    _compare("backward 2x3500x2", got, ref)


def test_backward_training_shape_every_head():
    """The training shape the benchmark times (8 sequences of 4096 tokens, 32
    heads, gated mix, no initial state), in the launch configuration it
    times: every gradient of every head against the oracle (eight heads per
    oracle call), and all of it finite."""
    import time
    dev = device()
    B, T, H = ki.BACKWARD_SHAPE
    inp = ki.workload_backward()
    d_o, d_s = ki.loss_gradients(ki.BACKWARD_WORKLOAD, (B, T, H, 128), B, H)
    got = _dense(inp, d_o, d_s, dev)
    for n, x in got.items():
        assert np.all(np.isfinite(x)), n
    wide = inp.widened()
    t0 = time.time()
    for h0 in range(0, H, 8):
        heads = list(range(h0, h0 + 8))
        q, k, v, b, la = (x[:, :, heads] for x in wide)
        ref = oracle.backward(q, k, v, b, la, d_o[:, :, heads], None, d_s[:, heads])
        sub = {n: (x[:, heads] if n == "dinitial_state" else x[:, :, heads]) for n, x in got.items()}
        _compare(f"backward 8x4096x32, heads {h0}..{h0 + 7}", sub, ref)
    print(f"oracle: {time.time() - t0:.1f} s for 32 heads", flush=True)


def test_backward_deterministic():
    """Two calls on the same inputs give the same bits (no atomics, fixed
    reduction order)."""
    torch = __import__("torch")
    dev = device()
    inp = ki.dense_prefill(53, B=2, T=77, H=3, gated=True, initial_state=True)
    d_o, d_s = ki.loss_gradients(53, (2, 77, 3, 128), 2, 3)
    t = upload(inp, dev)
    args = (t["q"], t["k"], t["v"], t["beta"], t["log_alpha"], to_dev(d_o, "f32", dev),
            t["initial_state"], to_dev(d_s, "f32", dev))
    g1 = kda.kda_backward(*args)
    g2 = kda.kda_backward(*args)
    torch.cuda.synchronize()
    for n in g1:
        assert torch.equal(g1[n], g2[n]), n


def test_backward_many_short_packed():
    """200 packed sequences of 0 to 40 tokens (seeded lengths; each within
    one chunk, a few empty, so most chunk ids start a sequence), two heads."""
    torch = __import__("torch")
    dev = device()
    lengths = [int(x) for x in np.random.default_rng(54).integers(0, 41, 200)]
    H = 2
    inp = ki.varlen_prefill(54, lengths, H=H)
    Tt = int(sum(lengths))
    d_o, d_s = ki.loss_gradients(54, (1, Tt, H, 128), len(lengths), H)
    t = upload(inp, dev)
    g = kda.kda_varlen_backward(t["q"], t["k"], t["v"], t["beta"], t["log_alpha"],
                                to_dev(d_o, "f32", dev), t["cu_seqlens"], t["initial_state"],
                                to_dev(d_s, "f32", dev))
    torch.cuda.synchronize()
    got = {n: (x.cpu().numpy()[0] if n != "dinitial_state" else x.cpu().numpy()) for n, x in g.items()}
    ref = oracle.varlen_backward(*inp.widened(), d_o, inp.cu_seqlens, inp.initial_state, d_s)
    _compare("backward 200 short packed sequences", got, ref)


@pytest.mark.parametrize("T", [30, 2100])
def test_backward_initial_gradient_in_place(T):
    """d_initial_state may be the d_final_state buffer itself (include/kda.h
    allows it: the final-state gradient is read before the initial one is
    written).  Called through the C ABI with one buffer for both: the same
    bits as separate buffers, in one chunk (30 tokens) and in 33 chunks
    (2100 tokens, two heads of one sequence)."""
    import ctypes
    torch = __import__("torch")
    dev = device()
    B, H = (2, 2) if T < 1000 else (1, 2)
    inp = ki.dense_prefill(55, B=B, T=T, H=H, gated=True, initial_state=True)
    d_o, d_s = ki.loss_gradients(55, (B, T, H, 128), B, H)
    t = upload(inp, dev)
    do = to_dev(d_o, "f32", dev)
    ref = kda.kda_backward(t["q"], t["k"], t["v"], t["beta"], t["log_alpha"], do,
                           t["initial_state"], to_dev(d_s, "f32", dev))
    buf = to_dev(d_s, "f32", dev)
    outs = {n: torch.empty_like(ref[n]) for n in ("dq", "dk", "dv", "dbeta", "dlog_alpha")}
    p = lambda x: ctypes.c_void_p(x.data_ptr())
    lib = kda.load_library()
    code = lib.kda_backward(p(t["q"]), p(t["k"]), p(t["v"]), p(t["beta"]), p(t["log_alpha"]),
                            p(t["initial_state"]), p(do), p(buf), p(outs["dq"]), p(outs["dk"]),
                            p(outs["dv"]), p(outs["dbeta"]), p(outs["dlog_alpha"]), p(buf),
                            B, T, H, 128, 128, kda.KDA_BF16, None, kda.KDA_WORKSPACE_AUTO,
                            ctypes.c_void_p(torch.cuda.current_stream(dev).cuda_stream))
    torch.cuda.synchronize()
    assert code == 0, code
    for n, x in outs.items():
        assert torch.equal(x, ref[n]), n
    assert torch.equal(buf, ref["dinitial_state"])
