"""Caller-owned workspaces, the library's opt-in pool, a pending HIP error
and the KDA_DEBUG precondition checks, on the GPU.

* A prefill or backward call gives the same bits whether its workspace is a
  caller tensor of the size the query reports, a larger caller tensor, or the
  library's own stream-ordered allocation (KDA_WORKSPACE_AUTO).
* A workspace of a smaller plan's size selects that plan (checked against the
  oracle); a backward workspace one byte short is refused with nothing
  enqueued.
* A HIP error the caller left unread is not cleared by the library.
* With KDA_DEBUG, out-of-range gates and malformed cu_seqlens are refused
  before any kernel reads them (in a child process, since the setting is read
  once per process)."""
import ctypes
import os
import subprocess
import sys

import numpy as np
import pytest

import gated_delta_rule_113_amd as kda
import kda_inputs as ki
import oracle
from kda_gpu import check, device, rel_err_states, rel_err_vectors, upload

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _torch():
    import torch
    return torch


def _bytes(n):
    torch = _torch()
    return torch.empty(max(n, 1), dtype=torch.uint8, device=device())


def test_dense_prefill_workspace_forms_agree():
    torch = _torch()
    inp = ki.dense_prefill(70, B=2, T=4096, H=8, gated=True, initial_state=True)
    t = upload(inp, device())
    sizes = [kda.prefill_workspace_size(2, 4096, 8, torch.bfloat16, p)
             for p in (kda.KDA_PLAN_FULL, kda.KDA_PLAN_SEGMENTS, kda.KDA_PLAN_UNSEGMENTED)]
    print("workspace bytes (full, segments, unsegmented):", sizes, flush=True)
    assert sizes[0] > sizes[1] > 0 and sizes[2] == 0

    def run(ws):
        o, S = kda.kda_prefill(t["q"], t["k"], t["v"], t["beta"], t["log_alpha"],
                               t["initial_state"], workspace=ws)
        torch.cuda.synchronize()
        return o.cpu().numpy(), S.cpu().numpy()

    o_none, S_none = run(None)
    o_auto, S_auto = run("auto")
    o_exact, S_exact = run(_bytes(sizes[0]))
    o_big, S_big = run(_bytes(sizes[0] + (1 << 20)))
    for o, S in ((o_auto, S_auto), (o_exact, S_exact), (o_big, S_big)):
        assert np.array_equal(o, o_none) and np.array_equal(S, S_none)
    o_ref, S_ref = oracle.prefill(*inp.widened(), inp.initial_state)
    check("workspace: full plan", rel_err_vectors(o_none, o_ref), rel_err_states(S_none, S_ref))
    # one byte short of the full plan: the segment plan without T/P images
    o_seg, S_seg = run(_bytes(sizes[0] - 1))
    o_seg2, S_seg2 = run(_bytes(sizes[1]))
    assert np.array_equal(o_seg, o_seg2) and np.array_equal(S_seg, S_seg2)
    check("workspace: segments plan", rel_err_vectors(o_seg, o_ref), rel_err_states(S_seg, S_ref))
    # below the segment plan: unsegmented, no workspace touched
    o_un, S_un = run(_bytes(sizes[1] - 1))
    o_un2, S_un2 = run(_bytes(0)[:0])
    assert np.array_equal(o_un, o_un2) and np.array_equal(S_un, S_un2)
    check("workspace: unsegmented plan", rel_err_vectors(o_un, o_ref), rel_err_states(S_un, S_ref))


def test_packed_prefill_workspace_forms_agree():
    torch = _torch()
    lengths = [0, 5, 3000, 17, 1500, 2600, 64, 900]
    inp = ki.varlen_prefill(71, lengths, H=6)
    t = upload(inp, device())
    Tt = int(inp.cu_seqlens[-1])
    full = kda.varlen_prefill_workspace_size(len(lengths), Tt, 6, torch.bfloat16)
    seg = kda.varlen_prefill_workspace_size(len(lengths), Tt, 6, torch.bfloat16, kda.KDA_PLAN_SEGMENTS)
    assert full > seg > 0

    def run(ws):
        o, S = kda.kda_varlen_prefill(t["q"], t["k"], t["v"], t["beta"], t["log_alpha"],
                                      t["cu_seqlens"], t["initial_state"], workspace=ws)
        torch.cuda.synchronize()
        return o.cpu().numpy(), S.cpu().numpy()

    o1, S1 = run(None)
    o2, S2 = run("auto")
    o3, S3 = run(_bytes(full))
    assert np.array_equal(o1, o2) and np.array_equal(S1, S2)
    assert np.array_equal(o1, o3) and np.array_equal(S1, S3)
    o_ref, S_ref = oracle.varlen_prefill(*inp.widened(), inp.cu_seqlens, inp.initial_state)
    check("packed workspace: full plan", rel_err_vectors(o1[0], o_ref), rel_err_states(S1, S_ref))
    o4, S4 = run(_bytes(seg))
    check("packed workspace: segments plan", rel_err_vectors(o4[0], o_ref), rel_err_states(S4, S_ref))
    o5, S5 = run(_bytes(0)[:0])
    check("packed workspace: unsegmented", rel_err_vectors(o5[0], o_ref), rel_err_states(S5, S_ref))


def test_backward_workspace_forms_agree_and_short_one_is_refused():
    torch = _torch()
    B, T, H = 2, 300, 3
    inp = ki.dense_prefill(72, B=B, T=T, H=H, gated=True, initial_state=True)
    d_o, d_s = ki.loss_gradients(72, (B, T, H, 128), B, H)
    t = upload(inp, device())
    do_t = torch.from_numpy(d_o).to(device())
    ds_t = torch.from_numpy(d_s).to(device())
    n = kda.backward_workspace_size(B, T, H, torch.bfloat16)
    assert n > 0

    def run(ws):
        g = kda.kda_backward(t["q"], t["k"], t["v"], t["beta"], t["log_alpha"], do_t,
                             t["initial_state"], ds_t, workspace=ws)
        torch.cuda.synchronize()
        return {k_: x.cpu().numpy() for k_, x in g.items()}

    g1, g2, g3 = run(None), run("auto"), run(_bytes(n))
    for g in (g2, g3):
        for name in g1:
            assert np.array_equal(g[name], g1[name]), name
    with pytest.raises(kda.KDAError) as err:
        run(_bytes(n - 1))
    assert err.value.code == 7   # KDA_ERR_WORKSPACE


def _hip_runtime():
    """The HIP runtime this process already uses (the one torch loaded)."""
    with open("/proc/self/maps") as f:
        for line in f:
            if "libamdhip64.so" in line:
                return ctypes.CDLL(line.split()[-1])
    pytest.skip("HIP runtime not found in the process maps")


def test_pending_hip_error_is_left_for_the_caller():
    """An unread HIP error (from an invalid hipSetDevice of the caller's)
    makes a call enqueue nothing and return KDA_ERR_HIP; the error is still
    there for the caller to read, and afterwards calls work again."""
    torch = _torch()
    hip = _hip_runtime()
    inp = ki.decode_steps(73, steps=1, N=2, H=2)
    t = upload(inp, device())
    state = t["initial_state"].clone()
    before = state.clone()
    torch.cuda.synchronize()
    # the runtime keeps an error across later successful calls until it is read
    assert hip.hipSetDevice(ctypes.c_int(4096)) != 0
    d = ctypes.c_int(-1)
    assert hip.hipGetDevice(ctypes.byref(d)) == 0
    if hip.hipPeekAtLastError() == 0:
        pytest.skip("this HIP runtime clears the last error on a successful call")
    assert hip.hipGetLastError() != 0 and hip.hipGetLastError() == 0
    assert hip.hipSetDevice(ctypes.c_int(4096)) != 0       # leaves an error pending
    with pytest.raises(kda.KDAError) as err:
        kda.kda_decode_step(t["q"][0], t["k"][0], t["v"][0], t["beta"][0], t["log_alpha"][0], state)
    assert err.value.code == 6
    assert hip.hipGetLastError() != 0                      # still pending, now read
    assert hip.hipGetLastError() == 0
    torch.cuda.synchronize()
    assert torch.equal(state, before)                      # nothing was enqueued
    kda.kda_decode_step(t["q"][0], t["k"][0], t["v"][0], t["beta"][0], t["log_alpha"][0], state)
    torch.cuda.synchronize()
    assert not torch.equal(state, before)


DEBUG_CHILD = r'''
import sys
sys.path.insert(0, sys.argv[1])
import torch
import gated_delta_rule_113_amd as kda
dev = torch.device("cuda", 0)
T, H = 80, 2
q = torch.zeros(1, T, H, 128, dtype=torch.bfloat16, device=dev)
beta = torch.zeros(1, T, H, dtype=torch.bfloat16, device=dev)
la = torch.full((1, T, H, 128), -0.1, device=dev)

def status(fn):
    try:
        fn()
        torch.cuda.synchronize()
        return 0
    except kda.KDAError as e:
        return e.code

ok = status(lambda: kda.kda_prefill(q, q, q, beta, la))
la_pos = la.clone(); la_pos[0, 7, 1, 3] = 0.5
pos = status(lambda: kda.kda_prefill(q, q, q, beta, la_pos))
la_nan = la.clone(); la_nan[0, 60, 0, 127] = float("nan")
nan = status(lambda: kda.kda_prefill(q, q, q, beta, la_nan))
raw_pos = status(lambda: kda.kda_prefill_raw(q, q, q, beta, la_pos))
la_inf = la.clone(); la_inf[0, 0, 0, 0] = float("-inf")
raw_inf = status(lambda: kda.kda_prefill_raw(q, q, q, beta, la_inf))
cu_ok = torch.tensor([0, 30, 80], dtype=torch.int32, device=dev)
cu_dec = torch.tensor([0, 50, 40, 80], dtype=torch.int32, device=dev)
cu_end = torch.tensor([0, 30, 79], dtype=torch.int32, device=dev)
cu_start = torch.tensor([1, 30, 80], dtype=torch.int32, device=dev)
v_ok = status(lambda: kda.kda_varlen_prefill(q, q, q, beta, la, cu_ok))
v_dec = status(lambda: kda.kda_varlen_prefill(q, q, q, beta, la, cu_dec))
v_end = status(lambda: kda.kda_varlen_prefill(q, q, q, beta, la, cu_end))
v_start = status(lambda: kda.kda_varlen_prefill(q, q, q, beta, la, cu_start))
print("STATUS", ok, pos, nan, raw_pos, raw_inf, v_ok, v_dec, v_end, v_start, flush=True)
'''


def test_debug_preconditions_refuse_bad_device_data():
    env = dict(os.environ, KDA_DEBUG="1")
    r = subprocess.run([sys.executable, "-c", DEBUG_CHILD, ROOT], env=env, capture_output=True,
                       text=True, timeout=240)
    print(r.stdout[-2000:], r.stderr[-2000:], flush=True)
    assert r.returncode == 0
    line = [l for l in r.stdout.splitlines() if l.startswith("STATUS")][-1]
    got = [int(x) for x in line.split()[1:]]
    PRE = 8
    #       ok  pos  nan  raw+ raw-inf v_ok v_dec v_end v_start
    assert got == [0, PRE, PRE, 0, PRE, 0, PRE, PRE, PRE]
