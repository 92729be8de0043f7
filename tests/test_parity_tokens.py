"""K draft tokens per sequence from its state (kda_decode_tokens) on the GPU:
outputs of all K tokens and the committed prefix state against the fp64
oracle, the state untouched without a commit, and agreement with a chain of
single-token decode steps."""
import numpy as np
import pytest

import gated_delta_rule_113_amd as kda
import kda_inputs as ki
import oracle
from kda_gpu import check, device, rel_err_states, rel_err_vectors, to_dev

pytestmark = pytest.mark.gpu


def _torch():
    import torch
    return torch


def _inputs(workload, N, K, H, dtype):
    """[N, K, H, *] token inputs (decode-step draws, token-major regrouped) and
    N(0, 0.02^2) states."""
    inp = ki.decode_steps(workload, steps=K, N=N, H=H, dtype=dtype)
    nk = lambda x: np.ascontiguousarray(np.swapaxes(x, 0, 1))
    return inp, {n: nk(getattr(inp, n)) for n in ("q", "k", "v", "beta", "log_alpha")}


def _upload(arrs, dtype, dev):
    return {n: to_dev(x, "f32" if n == "log_alpha" else dtype, dev) for n, x in arrs.items()}


def _oracle(inp, N, K, commit):
    """Outputs of all K tokens from the initial states, and each sequence's
    state after its first commit[n] tokens."""
    q, k, v, b, la = (np.ascontiguousarray(np.swapaxes(x, 0, 1)) for x in inp.widened())
    H = q.shape[2]
    flat = lambda x: x.reshape(N * K, H, *x.shape[3:])
    o, _ = oracle.run_rows(flat(q), flat(k), flat(v), flat(b), flat(la), np.arange(N) * K,
                           np.full(N, K), 1, inp.initial_state)
    _, S = oracle.run_rows(flat(q), flat(k), flat(v), flat(b), flat(la), np.arange(N) * K,
                           np.asarray(commit, np.int64), 1, inp.initial_state)
    return o.reshape(N, K, H, -1), S


@pytest.mark.parametrize("dtype,K,gates", [("bf16", 4, None), ("f32", 4, None), ("bf16", 1, None),
                                           ("bf16", 6, None), ("bf16", 16, None), ("f32", 16, None),
                                           ("bf16", 8, "extreme"), ("bf16", 3, "extreme"),
                                           ("f32", 2, None)])
def test_verify_then_commit(dtype, K, gates):
    torch = _torch()
    dev = device()
    N, H = 6, 3
    inp, arrs = _inputs(31, N, K, H, dtype)
    if gates == "extreme":
        # per channel: no decay, almost none, or decay that underflows within
        # a token (log alpha = -60, -200) -- the chunk form's factors
        # 2^(G_r - G_i) then span the whole fp32 range
        levels = np.array([0.0, -1e-3, -60.0, -200.0], np.float32)
        la = levels[np.random.default_rng(5).integers(0, 4, size=inp.log_alpha.shape)]
        inp = ki.KDAInputs(inp.q, inp.k, inp.v, inp.beta, la, inp.dtype, inp.initial_state)
        arrs["log_alpha"] = np.ascontiguousarray(np.swapaxes(la, 0, 1))
    t = _upload(arrs, dtype, dev)
    s0 = to_dev(inp.initial_state, "f32", dev)
    # verify: outputs of all K tokens, state only read
    state = s0.clone()
    o = kda.kda_decode_tokens(t["q"], t["k"], t["v"], t["beta"], t["log_alpha"], state)
    torch.cuda.synchronize()
    assert torch.equal(state, s0)
    # commit accepted prefixes; out-of-range counts are clamped to [0, K]
    accepted = np.array([0, 1, K, K // 2, K + 5, -3], np.int32)
    clamped = np.clip(accepted, 0, K)
    o2 = kda.kda_decode_tokens(t["q"], t["k"], t["v"], t["beta"], t["log_alpha"], state,
                               torch.from_numpy(accepted).to(dev))
    torch.cuda.synchronize()
    o, o2, S = o.cpu().numpy(), o2.cpu().numpy(), state.cpu().numpy()
    if K > 4:
        assert np.array_equal(o, o2)                # the commit pass recomputes the same bits
    else:
        # verify without a commit runs the streaming kernel, the commit call
        # the register-resident one: the same arithmetic, summed in another order
        assert rel_err_vectors(o, o2) < 1e-5
    o_ref, S_ref = _oracle(inp, N, K, clamped)
    check(f"decode tokens {dtype} K={K}", rel_err_vectors(o, o_ref), rel_err_states(S, S_ref))
    for n in np.nonzero(clamped == 0)[0]:           # nothing accepted: state unchanged
        assert np.array_equal(S[n], inp.initial_state[n])


def test_tokens_match_single_steps_full_size():
    """The batched decode shape (64 x 32 heads) with K = 4, verified and then
    every token committed, against four single-token decode steps and, for
    two heads, the oracle.  The two kernels run the same fp32 recurrence but form the output
    differently (read from the updated state here, as r + (k.q) u in the
    decode step), so they agree to fp32 rounding, not bit for bit."""
    torch = _torch()
    dev = device()
    N, H, K = 64, 32, 4
    inp, arrs = _inputs(32, N, K, H, "bf16")
    t = _upload(arrs, "bf16", dev)
    state = to_dev(inp.initial_state, "f32", dev)
    o_verify = kda.kda_decode_tokens(t["q"], t["k"], t["v"], t["beta"], t["log_alpha"], state)
    o = kda.kda_decode_tokens(t["q"], t["k"], t["v"], t["beta"], t["log_alpha"], state,
                              torch.full((N,), K, dtype=torch.int32, device=dev))
    chain = to_dev(inp.initial_state, "f32", dev)
    steps = [kda.kda_decode_step(t["q"][:, s].contiguous(), t["k"][:, s].contiguous(),
                                 t["v"][:, s].contiguous(), t["beta"][:, s].contiguous(),
                                 t["log_alpha"][:, s].contiguous(), chain) for s in range(K)]
    torch.cuda.synchronize()
    o, o_verify = o.cpu().numpy(), o_verify.cpu().numpy()
    o_steps = torch.stack(steps, dim=1).cpu().numpy()
    S, S_chain = state.cpu().numpy(), chain.cpu().numpy()
    assert rel_err_vectors(o, o_steps) < 1e-5 and rel_err_states(S, S_chain) < 1e-6
    assert rel_err_vectors(o_verify, o_steps) < 1e-5
    sub = _inputs(32, N, K, H, "bf16")[0]
    heads = [0, 31]
    sub = ki.KDAInputs(*(getattr(sub, n)[:, :, heads] for n in ("q", "k", "v", "beta", "log_alpha")),
                       "bf16", sub.initial_state[:, heads])
    o_ref, S_ref = _oracle(sub, N, K, np.full(N, K))
    check("decode tokens full size, heads 0 and 31", rel_err_vectors(o[:, :, heads], o_ref),
          rel_err_states(S[:, heads], S_ref))


@pytest.mark.parametrize("K", [4, 6])
def test_tokens_streamed_state_every_head(K):
    """A batch whose states (136 sequences x 32 heads, 272 MiB) exceed the
    256 MB last-level cache, which the kernels stream with the nontemporal
    hint: verify (K = 4 takes the streaming verify kernel), then commit of
    per-sequence prefixes of 0..K tokens; every head against the oracle."""
    torch = _torch()
    dev = device()
    N, H = 136, 32
    inp, arrs = _inputs(33, N, K, H, "bf16")
    t = _upload(arrs, "bf16", dev)
    s0 = to_dev(inp.initial_state, "f32", dev)
    state = s0.clone()
    o = kda.kda_decode_tokens(t["q"], t["k"], t["v"], t["beta"], t["log_alpha"], state)
    torch.cuda.synchronize()
    assert torch.equal(state, s0)
    del s0
    accepted = (np.arange(N) % (K + 1)).astype(np.int32)
    o2 = kda.kda_decode_tokens(t["q"], t["k"], t["v"], t["beta"], t["log_alpha"], state,
                               torch.from_numpy(accepted).to(dev))
    torch.cuda.synchronize()
    o, o2, S = o.cpu().numpy(), o2.cpu().numpy(), state.cpu().numpy()
    o_ref, S_ref = _oracle(inp, N, K, accepted)
    check(f"decode tokens streamed state K={K}, verify", rel_err_vectors(o, o_ref), rel_err_states(S, S_ref))
    check(f"decode tokens streamed state K={K}, commit", rel_err_vectors(o2, o_ref), rel_err_states(S, S_ref))
