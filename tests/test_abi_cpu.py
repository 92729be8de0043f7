"""The C ABI on the CPU: the library loads, exports every function that
include/kda.h declares, and rejects bad arguments before any launch.

No call here reaches a kernel: every call carries an argument the host-side
validation refuses (pointers are fake, never dereferenced)."""
import ctypes
import os
import re
import subprocess

import pytest

import gated_delta_rule_113_amd as kda

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "kda.h")

OK, NULL, SHAPE, DTYPE, ALIGN, UNSUP, HIP, WORKSPACE, PRECONDITION, OVERLAP = range(10)
AUTO = -1            # KDA_WORKSPACE_AUTO
P = 0x10000          # a 16-byte aligned fake device address
MIS = 0x10008        # 8-byte aligned only


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(kda._binding.LIBRARY):
        from gated_delta_rule_113_amd import build
        build.build()
    return kda.load_library()


def _declared():
    with open(HEADER) as f:
        text = f.read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return set(re.findall(r"\b(kda_[a-z_]+)\s*\(", text))


def test_exports_match_header(lib):
    declared = _declared()
    assert declared == {"kda_prefill", "kda_prefill_noalloc", "kda_varlen_prefill", "kda_decode_step",
                        "kda_prefill_raw", "kda_varlen_prefill_raw", "kda_decode_step_raw",
                        "kda_decode_tokens", "kda_decode_step_slots", "kda_varlen_prefill_slots",
                        "kda_backward", "kda_varlen_backward", "kda_prefill_workspace_size",
                        "kda_varlen_prefill_workspace_size", "kda_backward_workspace_size",
                        "kda_varlen_backward_workspace_size", "kda_set_prefill_segment",
                        "kda_status_str", "kda_abi_version"}
    out = subprocess.run(["nm", "-D", "--defined-only", kda._binding.LIBRARY],
                         capture_output=True, text=True, check=True).stdout
    exported = set(re.findall(r" T (kda_\w+)", out))
    assert declared <= exported, declared - exported
    for name in declared:
        assert hasattr(lib, name)
    assert set(kda.EXPORTS) == declared


def test_version_and_status_strings(lib):
    assert lib.kda_abi_version() == 3
    for code in range(10):
        s = lib.kda_status_str(code).decode()
        assert s.startswith(kda._binding.STATUS_NAMES[code])
    assert lib.kda_status_str(99).decode().startswith("KDA_ERR_UNKNOWN")


def prefill(lib, q=P, k=P, v=P, beta=P, la=P, s0=None, o=P, s1=P, B=1, T=4, H=2,
            dk=128, dv=128, dt=1, ws=None, wb=0):
    return lib.kda_prefill(q, k, v, beta, la, s0, o, s1, B, T, H, dk, dv, dt, ws, wb, None)


def varlen(lib, q=P, k=P, v=P, beta=P, la=P, cu=P, N=2, Tt=8, s0=None, o=P, s1=P, H=2,
           dk=128, dv=128, dt=1, ws=None, wb=0):
    return lib.kda_varlen_prefill(q, k, v, beta, la, cu, N, Tt, s0, o, s1, H, dk, dv, dt, ws, wb,
                                  None)


def decode(lib, q=P, k=P, v=P, beta=P, la=P, st=P, o=P, N=2, H=2, dk=128, dv=128, dt=1):
    return lib.kda_decode_step(q, k, v, beta, la, st, o, N, H, dk, dv, dt, None)


def test_prefill_validation(lib):
    assert prefill(lib, q=None) == NULL
    assert prefill(lib, o=None) == NULL
    assert prefill(lib, la=None) == NULL
    assert prefill(lib, k=MIS) == ALIGN
    assert prefill(lib, s0=MIS) == ALIGN
    assert prefill(lib, s1=MIS) == ALIGN
    assert prefill(lib, dk=64) == UNSUP
    assert prefill(lib, dv=256) == UNSUP
    assert prefill(lib, dk=0) == SHAPE
    assert prefill(lib, H=0) == SHAPE
    assert prefill(lib, H=65537, T=1) == SHAPE   # in-chunk offsets are 32-bit
    assert prefill(lib, B=-1) == SHAPE
    assert prefill(lib, T=-5) == SHAPE
    assert prefill(lib, T=1 << 40) == SHAPE
    assert prefill(lib, dt=2) == DTYPE
    assert prefill(lib, dt=-1) == DTYPE
    # B = 0 is a no-op and needs no pointers at all
    assert prefill(lib, B=0, q=None, k=None, v=None, beta=None, la=None, o=None, s1=None) == OK
    # T = 0 without a final state has nothing to write
    assert prefill(lib, T=0, q=None, k=None, v=None, beta=None, la=None, o=None, s1=None) == OK


def test_noalloc_validates_like_the_plain_call(lib):
    """kda_prefill_noalloc refuses what kda_prefill refuses, before it looks up
    its scratch on the device."""
    def noalloc(q=P, k=P, v=P, beta=P, la=P, s0=None, o=P, s1=P, B=1, T=4, H=2, dk=128, dv=128, dt=1):
        return lib.kda_prefill_noalloc(q, k, v, beta, la, s0, o, s1, B, T, H, dk, dv, dt, None)
    for kw, expect in (({"q": None}, NULL), ({"o": None}, NULL), ({"k": MIS}, ALIGN),
                       ({"s1": MIS}, ALIGN), ({"dk": 64}, UNSUP), ({"dt": 2}, DTYPE), ({"H": 0}, SHAPE),
                       ({"B": -1}, SHAPE), ({"T": 1 << 40}, SHAPE)):
        assert noalloc(**kw) == expect, kw
        assert prefill(lib, **kw) == expect, kw
    assert noalloc(B=0, q=None, o=None, s1=None) == OK


def test_raw_entry_points_validate_like_the_plain_ones(lib):
    for fn_plain, fn_raw in (("kda_prefill", "kda_prefill_raw"),
                             ("kda_varlen_prefill", "kda_varlen_prefill_raw"),
                             ("kda_decode_step", "kda_decode_step_raw")):
        plain, raw = getattr(lib, fn_plain), getattr(lib, fn_raw)
        lib_alias = type("L", (), {fn_plain: raw})
        call = {"kda_prefill": prefill, "kda_varlen_prefill": varlen, "kda_decode_step": decode}[fn_plain]
        for kw, expect in (({"q": None}, NULL), ({"k": MIS}, ALIGN), ({"dk": 64}, UNSUP),
                           ({"dt": 2}, DTYPE), ({"H": 0}, SHAPE)):
            assert call(lib_alias, **kw) == expect, (fn_raw, kw)
            assert call(lib, **kw) == expect, (fn_plain, kw)


def test_varlen_validation(lib):
    assert varlen(lib, cu=None) == NULL
    assert varlen(lib, cu=P + 4) == ALIGN
    assert varlen(lib, v=None) == NULL
    assert varlen(lib, N=-1) == SHAPE
    assert varlen(lib, Tt=-1) == SHAPE
    assert varlen(lib, Tt=1 << 31) == SHAPE     # cu_seqlens holds int32 offsets
    assert varlen(lib, dk=96) == UNSUP
    assert varlen(lib, H=65537) == SHAPE
    assert varlen(lib, dt=7) == DTYPE
    assert varlen(lib, N=0, cu=None, q=None, o=None) == OK
    assert varlen(lib, Tt=0, q=None, k=None, v=None, beta=None, la=None, o=None, s1=None) == OK


def test_decode_validation(lib):
    for name in ("q", "k", "v", "beta", "la", "st", "o"):
        assert decode(lib, **{name: None}) == NULL, name
        assert decode(lib, **{name: MIS}) == ALIGN, name
    assert decode(lib, N=-3) == SHAPE
    assert decode(lib, H=0) == SHAPE
    assert decode(lib, H=65537) == SHAPE
    assert decode(lib, dk=127) == UNSUP
    assert decode(lib, dt=3) == DTYPE
    assert decode(lib, N=0, q=None) == OK


def decode_slots(lib, q=P, k=P, v=P, beta=P, la=P, pool=P, slots=P, n_pool=4, o=P, N=2, H=2,
                 dk=128, dv=128, dt=1):
    return lib.kda_decode_step_slots(q, k, v, beta, la, pool, slots, n_pool, o, N, H, dk, dv, dt,
                                     None)


def varlen_slots(lib, q=P, k=P, v=P, beta=P, la=P, cu=P, N=2, Tt=8, pool=P, si=P, sf=P, n_pool=4,
                 o=P, H=2, dk=128, dv=128, dt=1):
    return lib.kda_varlen_prefill_slots(q, k, v, beta, la, cu, N, Tt, pool, si, sf, n_pool, o, H,
                                        dk, dv, dt, None, 0, None)


def decode_tokens(lib, q=P, k=P, v=P, beta=P, la=P, st=P, nc=None, o=P, N=2, K=4, H=2, dk=128,
                  dv=128, dt=1):
    return lib.kda_decode_tokens(q, k, v, beta, la, st, nc, o, N, K, H, dk, dv, dt, None)


def test_decode_tokens_validation(lib):
    for name in ("q", "k", "v", "beta", "la", "st", "o"):
        assert decode_tokens(lib, **{name: None}) == NULL, name
        assert decode_tokens(lib, **{name: MIS}) == ALIGN, name
    assert decode_tokens(lib, nc=MIS) == ALIGN
    assert decode_tokens(lib, K=0) == SHAPE
    assert decode_tokens(lib, K=17) == SHAPE       # at most 16 draft tokens
    assert decode_tokens(lib, N=-1) == SHAPE
    assert decode_tokens(lib, dk=16) == UNSUP
    assert decode_tokens(lib, dt=4) == DTYPE
    assert decode_tokens(lib, N=0, q=None, st=None) == OK


def test_decode_slots_validation(lib):
    for name in ("q", "k", "v", "beta", "la", "pool", "slots", "o"):
        assert decode_slots(lib, **{name: None}) == NULL, name
        assert decode_slots(lib, **{name: MIS}) == ALIGN, name
    assert decode_slots(lib, N=-1) == SHAPE
    assert decode_slots(lib, n_pool=-1) == SHAPE
    assert decode_slots(lib, n_pool=1 << 40) == SHAPE   # pool index products overflow
    assert decode_slots(lib, H=0) == SHAPE
    assert decode_slots(lib, dv=64) == UNSUP
    assert decode_slots(lib, dt=5) == DTYPE
    assert decode_slots(lib, N=0, q=None, pool=None, slots=None) == OK


def test_varlen_slots_validation(lib):
    assert varlen_slots(lib, cu=None) == NULL
    assert varlen_slots(lib, pool=None) == NULL             # slots need a pool
    assert varlen_slots(lib, si=MIS) == ALIGN
    assert varlen_slots(lib, sf=MIS) == ALIGN
    assert varlen_slots(lib, n_pool=-2) == SHAPE
    assert varlen_slots(lib, Tt=-1) == SHAPE
    assert varlen_slots(lib, dk=32) == UNSUP
    assert varlen_slots(lib, dt=9) == DTYPE
    assert varlen_slots(lib, N=0, cu=None, pool=None) == OK
    # nothing to read and nothing to write
    assert varlen_slots(lib, Tt=0, pool=None, si=None, sf=None, q=None, o=None) == OK


def backward(lib, q=P, k=P, v=P, beta=P, la=P, s0=None, do=P, dsT=None, dq=P, dk_=P, dv_=P, db=P,
             dla=P, ds0=P, B=1, T=4, H=2, dk=128, dv=128, dt=1, ws=None, wb=0):
    return lib.kda_backward(q, k, v, beta, la, s0, do, dsT, dq, dk_, dv_, db, dla, ds0,
                            B, T, H, dk, dv, dt, ws, wb, None)


def varlen_backward(lib, q=P, k=P, v=P, beta=P, la=P, cu=P, N=2, Tt=8, s0=None, do=P, dsT=None,
                    dq=P, dk_=P, dv_=P, db=P, dla=P, ds0=P, H=2, dk=128, dv=128, dt=1, ws=None,
                    wb=0):
    return lib.kda_varlen_backward(q, k, v, beta, la, cu, N, Tt, s0, do, dsT, dq, dk_, dv_, db,
                                   dla, ds0, H, dk, dv, dt, ws, wb, None)


def test_backward_validation(lib):
    for name in ("q", "k", "v", "beta", "la", "do", "dq", "dk_", "dv_", "db", "dla"):
        assert backward(lib, **{name: None}) == NULL, name
        assert backward(lib, **{name: MIS}) == ALIGN, name
        assert varlen_backward(lib, **{name: None}) == NULL, name
    for name in ("s0", "dsT", "ds0"):
        assert backward(lib, **{name: MIS}) == ALIGN, name
        assert varlen_backward(lib, **{name: MIS}) == ALIGN, name
    assert backward(lib, B=-1) == SHAPE
    assert backward(lib, T=-1) == SHAPE
    assert backward(lib, T=1 << 40) == SHAPE
    assert backward(lib, H=0) == SHAPE
    assert backward(lib, H=65537) == SHAPE
    assert backward(lib, dk=64) == UNSUP
    assert backward(lib, dt=2) == DTYPE
    assert varlen_backward(lib, cu=None) == NULL
    assert varlen_backward(lib, cu=P + 4) == ALIGN
    assert varlen_backward(lib, Tt=1 << 31) == SHAPE
    assert varlen_backward(lib, N=-1) == SHAPE
    assert varlen_backward(lib, dv=32) == UNSUP
    # no sequences: nothing to do and no pointers needed
    assert backward(lib, B=0, q=None, do=None, dq=None, ds0=None) == OK
    assert varlen_backward(lib, N=0, cu=None, q=None, do=None, dq=None, ds0=None) == OK
    # no tokens and no initial-state gradient requested: nothing to write
    none = dict(q=None, k=None, v=None, beta=None, la=None, do=None, dq=None, dk_=None,
                dv_=None, db=None, dla=None, ds0=None)
    assert backward(lib, T=0, **none) == OK
    assert varlen_backward(lib, Tt=0, **none) == OK


def test_backward_overlap(lib):
    # buffers 1 MiB apart (B=1, T=4, H=2 needs at most 128 KiB each); with no
    # overlap the call still stops before any launch: no workspace was given
    # (KDA_ERR_WORKSPACE), or without a GPU the runtime check (KDA_ERR_HIP)
    names = ("q", "k", "v", "beta", "la", "s0", "do", "dsT", "dq", "dk_", "dv_", "db", "dla", "ds0")
    apart = {n: (i + 1) << 20 for i, n in enumerate(names)}
    assert backward(lib, **apart) in (WORKSPACE, HIP)
    assert backward(lib, **dict(apart, ds0=apart["dsT"])) in (WORKSPACE, HIP)   # allowed alias
    assert backward(lib, **dict(apart, dq=apart["q"])) == OVERLAP
    assert backward(lib, **dict(apart, dv_=apart["v"] + 1024)) == OVERLAP   # partly over v (2 KiB of bf16)
    assert backward(lib, **dict(apart, dla=apart["dk_"])) == OVERLAP
    assert backward(lib, **dict(apart, db=apart["do"] + 4096 - 16)) == OVERLAP
    assert backward(lib, **dict(apart, ds0=apart["s0"])) == OVERLAP
    assert backward(lib, **dict(apart, dq=apart["q"] + 2048)) in (WORKSPACE, HIP)  # just past bf16 q
    vb = {n: (i + 1) << 20 for i, n in enumerate(names) if n not in ("s0", "dsT", "ds0")}
    assert varlen_backward(lib, **dict(vb, cu=P, s0=None, dsT=None, ds0=None, dq=vb["la"])) == OVERLAP


def test_binding_rejects_cpu_tensors(lib):
    torch = pytest.importorskip("torch")
    x = torch.zeros(1, 2, 1, 128)
    with pytest.raises(ValueError, match="GPU"):
        kda.kda_prefill(x, x, x, torch.zeros(1, 2, 1), x)


def test_binding_fails_loudly_without_library(tmp_path):
    with pytest.raises(ImportError, match="build"):
        kda.load_library(str(tmp_path / "libkda.so"))


def test_prefill_segment_knob(lib):
    """The segment-length knob accepts 0 and positive multiples of 64 only."""
    assert lib.kda_set_prefill_segment(64) == OK
    assert lib.kda_set_prefill_segment(4096) == OK
    assert lib.kda_set_prefill_segment(0) == OK
    assert lib.kda_set_prefill_segment(100) == SHAPE
    assert lib.kda_set_prefill_segment(-64) == SHAPE


W = 0x20000          # a 256-byte aligned fake workspace address


def test_workspace_arguments(lib):
    """Workspace rules, checked before anything reaches the device: a caller
    workspace is 256-byte aligned and non-NULL when it has bytes;
    KDA_WORKSPACE_AUTO takes no pointer; other negative sizes are refused."""
    for call in (prefill, varlen, backward, varlen_backward):
        assert call(lib, q=None, ws=W, wb=1 << 20) == NULL, call.__name__   # still validated first
        assert call(lib, ws=None, wb=4096) == NULL, call.__name__
        assert call(lib, ws=P + 16, wb=4096) == ALIGN, call.__name__        # 16- but not 256-aligned
        assert call(lib, ws=W, wb=AUTO) == WORKSPACE, call.__name__
        assert call(lib, ws=None, wb=-2) == WORKSPACE, call.__name__
        assert call(lib, ws=W, wb=-5) == WORKSPACE, call.__name__
    # no work: a workspace argument of any valid form is accepted
    assert prefill(lib, B=0, q=None, o=None, s1=None, ws=None, wb=AUTO) == OK
    assert varlen(lib, N=0, cu=None, q=None, o=None, ws=W, wb=256) == OK


def size_query(lib, fn, *args):
    out = ctypes.c_int64(-7)
    code = getattr(lib, fn)(*args, ctypes.byref(out))
    return code, out.value


def test_backward_workspace_bytes(lib):
    """The backward's workspace as the header states it: bf16, 176 KiB per
    (64-token chunk id, head) -- the entering state and the leaving-state
    gradient (2 x 64 KiB) and A, P, T (3 x 16 KiB) -- with ids below
    rows / 64 + sequences + 1; fp32, one 64 KiB state per 8 tokens of each
    sequence (dense) or fewer than T_total / 8 + N blocks (packed)."""
    per_chunk = (2 * 128 * 128 + 3 * 64 * 64) * 4
    assert per_chunk == 176 * 1024
    for B, T, H in ((8, 4096, 32), (1, 1048576, 32), (3, 100, 5), (1, 17, 1)):
        ids = B * T // 64 + B + 1
        assert size_query(lib, "kda_backward_workspace_size", B, T, H, 128, 128, 1) == (OK, ids * H * per_chunk)
        blocks = B * ((T + 7) // 8)
        assert size_query(lib, "kda_backward_workspace_size", B, T, H, 128, 128, 0) == (OK, blocks * H * 65536)
    for N, Tt, H in ((16, 360769, 32), (2000, 2000 * 37, 4)):
        ids = Tt // 64 + N + 1
        assert size_query(lib, "kda_varlen_backward_workspace_size", N, Tt, H, 128, 128, 1) == \
            (OK, ids * H * per_chunk)
        assert size_query(lib, "kda_varlen_backward_workspace_size", N, Tt, H, 128, 128, 0) == \
            (OK, (Tt // 8 + N) * H * 65536)
    # the training shape and the million-token shape of the header's figures
    assert size_query(lib, "kda_backward_workspace_size", 8, 4096, 32, 128, 128, 1)[1] / 2 ** 30 < 2.8
    assert size_query(lib, "kda_backward_workspace_size", 1, 1 << 20, 32, 128, 128, 1)[1] / 2 ** 30 < 88.1


def test_workspace_size_validation(lib):
    """The size queries validate like the calls and report 0 bytes then;
    fp32 inputs and bf16 sequences of at most 16 tokens (token-by-token
    kernel) need no workspace, known without a device."""
    bad_shapes = ((1, 4, 0, 128, 128, 1), (-1, 4, 2, 128, 128, 1), (1, 4, 2, 64, 128, 1),
                  (1, 4, 2, 128, 128, 3), (1, 1 << 40, 2, 128, 128, 1), (1, 4, 65537, 128, 128, 1))
    expect = (SHAPE, SHAPE, UNSUP, DTYPE, SHAPE, SHAPE)
    for args, code in zip(bad_shapes, expect):
        assert size_query(lib, "kda_prefill_workspace_size", *args, 0) == (code, 0), args
        assert size_query(lib, "kda_backward_workspace_size", *args) == (code, 0), args
    assert size_query(lib, "kda_varlen_prefill_workspace_size", 2, 1 << 31, 2, 128, 128, 1, 0)[0] == SHAPE
    assert size_query(lib, "kda_prefill_workspace_size", 1, 4, 2, 128, 128, 1, 3)[0] == SHAPE  # plan
    assert lib.kda_prefill_workspace_size(1, 4, 2, 128, 128, 1, 0, None) == NULL
    # no workspace without the chunked kernel: fp32 inputs, or at most 16 tokens
    for plan in (0, 1, 2):
        assert size_query(lib, "kda_prefill_workspace_size", 4, 50000, 32, 128, 128, 0, plan) == (OK, 0)
        assert size_query(lib, "kda_prefill_workspace_size", 4, 16, 32, 128, 128, 1, plan) == (OK, 0)
        assert size_query(lib, "kda_varlen_prefill_workspace_size", 3, 16, 8, 128, 128, 1, plan) == (OK, 0)
        assert size_query(lib, "kda_prefill_workspace_size", 0, 5000, 2, 128, 128, 1, plan) == (OK, 0)
