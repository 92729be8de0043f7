"""Million-token prefill on the GPU vs the fp64 oracle.

The workload: B = 1, H = 32, T = 1,048,576, bf16 q/k/v/beta, fp32 log_alpha
and state, the gated channel mix, zero initial state.  The check follows the
workload's own plan: (i) the GPU runs all 1,048,576 tokens and the oracle
recomputes heads 0 and 31 over all of them (outputs and final states); (ii) a
separate GPU prefill of the first 65,536 tokens is compared with the oracle on
the final states of all 32 heads.

The inputs take about 56 GiB of host and device memory; generating them and
running the oracle dominate the test's time."""
import time

import numpy as np
import pytest

import gated_delta_rule_113_amd as kda
import kda_inputs as ki
import oracle
from kda_gpu import check, device, rel_err_states, rel_err_vectors, to_dev

pytestmark = [pytest.mark.gpu, pytest.mark.slow]

T_FULL = 1 << 20
PREFIX = 65536
HEADS = (0, 31)


def _log(msg):
    print(f"[million] {msg}", flush=True)


def test_million_token_prefill():
    torch = __import__("torch")
    dev = device()
    t0 = time.time()
    inp = ki.workload_million()
    _log(f"inputs generated in {time.time() - t0:.0f}s")
    t = {n: to_dev(getattr(inp, n), "bf16", dev) for n in ("q", "k", "v", "beta")}
    t["log_alpha"] = to_dev(inp.log_alpha, "f32", dev)

    def widened(index):
        """Oracle inputs (exact fp32 widening) of a slice of the workload."""
        w = [ki.bf16_to_f32(np.ascontiguousarray(getattr(inp, n)[index]))
             for n in ("q", "k", "v", "beta")]
        return (*w, np.ascontiguousarray(inp.log_alpha[index]))

    # (i) all tokens; heads 0 and 31 checked over every token
    o, S = kda.kda_prefill(t["q"], t["k"], t["v"], t["beta"], t["log_alpha"], None)
    torch.cuda.synchronize()
    _log(f"GPU prefill of {T_FULL} tokens done")
    hs = list(HEADS)
    o_h = o[:, :, hs].cpu().numpy()
    S_h = S[:, hs].cpu().numpy()
    assert bool(torch.isfinite(o).all()) and bool(torch.isfinite(S).all())
    del o
    t1 = time.time()
    o_ref, S_ref = oracle.prefill(*widened((slice(None), slice(None), hs)), None)
    _log(f"oracle, 2 heads x {T_FULL} tokens, in {time.time() - t1:.0f}s")
    check("million, heads 0 and 31", rel_err_vectors(o_h, o_ref), rel_err_states(S_h, S_ref))

    # (ii) the 65,536-token prefix; final states of all heads
    pre = {n: x[:, :PREFIX].contiguous() for n, x in t.items()}
    del t
    o_p, S_p = kda.kda_prefill(pre["q"], pre["k"], pre["v"], pre["beta"], pre["log_alpha"], None)
    torch.cuda.synchronize()
    t2 = time.time()
    _, S_pref = oracle.prefill(*widened((slice(None), slice(0, PREFIX))), None)
    _log(f"oracle, 32 heads x {PREFIX} tokens, in {time.time() - t2:.0f}s")
    check("million prefix, all heads (final states)", 0.0, rel_err_states(S_p.cpu().numpy(), S_pref))
