"""kda_prefill_noalloc (the prefill whose workspace is the library's fixed
scratch array) through the C ABI against kda_prefill with a caller
workspace of the same size: the same plan, so the same bits, on two calls in
a row (the second smaller, over the scratch the first left behind); both
against the oracle; and the refusal of a problem too large for the scratch."""
import ctypes

import numpy as np
import pytest

import gated_delta_rule_113_amd as kda
import kda_inputs as ki
import oracle
from kda_gpu import check, device, rel_err_states, rel_err_vectors, upload

pytestmark = pytest.mark.gpu

SCRATCH = 160 << 20


def _p(x):
    return ctypes.c_void_p(None if x is None else x.data_ptr())


def _noalloc(t, B, T, H):
    torch = __import__("torch")
    dev = device()
    o = torch.full((B, T, H, 128), 7.0, dtype=torch.float32, device=dev)
    S = torch.full((B, H, 128, 128), 7.0, dtype=torch.float32, device=dev)
    lib = kda.load_library()
    code = lib.kda_prefill_noalloc(_p(t["q"]), _p(t["k"]), _p(t["v"]), _p(t["beta"]), _p(t["log_alpha"]),
                                   _p(t["initial_state"]), _p(o), _p(S), B, T, H, 128, 128, kda.KDA_BF16,
                                   ctypes.c_void_p(torch.cuda.current_stream(dev).cuda_stream))
    return code, o, S


def test_noalloc_matches_prefill_on_two_calls():
    torch = __import__("torch")
    dev = device()
    ws = torch.empty(SCRATCH, dtype=torch.uint8, device=dev)
    cases = [(80, 1, 8192, 32, False), (81, 2, 3000, 4, True)]   # the second is smaller
    for seed, B, T, H, resumed in cases:
        inp = ki.dense_prefill(seed, B=B, T=T, H=H, gated=True, initial_state=resumed)
        t = upload(inp, dev)
        full = kda.prefill_workspace_size(B, T, H, torch.bfloat16, kda.KDA_PLAN_FULL)
        seg = kda.prefill_workspace_size(B, T, H, torch.bfloat16, kda.KDA_PLAN_SEGMENTS)
        print(f"B={B} T={T} H={H}: full plan {full / 2**20:.1f} MiB, segments {seg / 2**20:.1f} MiB",
              flush=True)
        assert 0 < seg <= SCRATCH
        code, o, S = _noalloc(t, B, T, H)
        assert code == 0, kda._binding.STATUS_NAMES.get(code, code)
        o_ref_gpu, S_ref_gpu = kda.kda_prefill(t["q"], t["k"], t["v"], t["beta"], t["log_alpha"],
                                               t["initial_state"], workspace=ws)
        torch.cuda.synchronize()
        assert torch.equal(o, o_ref_gpu) and torch.equal(S, S_ref_gpu)
        o_ref, S_ref = oracle.prefill(*inp.widened(), inp.initial_state)
        check(f"noalloc B={B} T={T} H={H}", rel_err_vectors(o.cpu().numpy(), o_ref),
              rel_err_states(S.cpu().numpy(), S_ref))


def test_noalloc_refuses_what_the_scratch_cannot_hold():
    torch = __import__("torch")
    inp = ki.dense_prefill(82, B=1, T=8192, H=32)
    t = upload(inp, device())
    kda.kda_set_prefill_segment(64)        # 128 segments per head: 768 MiB of segment maps
    try:
        seg = kda.prefill_workspace_size(1, 8192, 32, torch.bfloat16, kda.KDA_PLAN_SEGMENTS)
        assert seg > SCRATCH
        code, o, S = _noalloc(t, 1, 8192, 32)
        torch.cuda.synchronize()
    finally:
        kda.kda_set_prefill_segment(0)
    assert code == 7                        # KDA_ERR_WORKSPACE
    assert bool((o == 7.0).all()) and bool((S == 7.0).all())   # nothing was enqueued
