"""Host builds under AddressSanitizer and UndefinedBehaviorSanitizer.

* The fp64 oracle (oracle/kda_oracle.c) with a small C driver that runs its
  three entry points on seeded inputs (packed sequences of lengths 0 to 129,
  with and without initial states and read-out magnitudes, the input
  preparation) and its refusals of bad sizes.  The driver writes every input
  and output; the plain oracle build must give the same results bit for bit.
* The C ABI's host code (kda_api.cpp, kda_runtime.cpp, kda_plan.cpp) with a
  C++ driver that checks argument validation, workspace rules, size queries
  up to the largest accepted shapes and the work plans' invariants.  The HIP
  kernels are linked from the regular build (their host part is launch code
  only); no call reaches a kernel, so no GPU is needed.

Both drivers stop at the first sanitizer report (-fno-sanitize-recover).
"""
import glob
import os
import shutil
import subprocess

import numpy as np
import pytest

import oracle

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HERE = os.path.join(ROOT, "tests", "sanitize")
CSRC = os.path.join(ROOT, "gated_delta_rule_113_amd", "csrc")
SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer"]
ENV = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:verify_asan_link_order=0",
           UBSAN_OPTIONS="print_stacktrace=1")


def _run(cmd, **kw):
    r = subprocess.run(cmd, capture_output=True, text=True, **kw)
    assert r.returncode == 0, f"{' '.join(cmd)}\n{r.stdout}\n{r.stderr}"
    return r


def _records(path):
    kinds = {0: np.float32, 1: np.float64, 2: np.int64}
    out = []
    with open(path, "rb") as f:
        while True:
            head = f.read(12)
            if not head:
                return out
            count = int(np.frombuffer(head[:8], np.int64)[0])
            kind = int(np.frombuffer(head[8:], np.int32)[0])
            dt = kinds[kind]
            out.append(np.frombuffer(f.read(count * np.dtype(dt).itemsize), dt))


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc is needed")
def test_oracle_under_sanitizers(tmp_path):
    exe = str(tmp_path / "oracle_driver")
    _run(["gcc", "-O1", "-g", "-std=c99", "-fopenmp"] + SAN +
         ["-o", exe, os.path.join(HERE, "oracle_driver.c"), oracle.SOURCE, "-lm"])
    data = str(tmp_path / "oracle.bin")
    r = _run([exe, data], env=ENV)
    assert "oracle driver done" in r.stdout
    recs = _records(data)
    pos = 0

    def take(n=1):
        nonlocal pos
        got = recs[pos:pos + n]
        pos += n
        return got

    for _case in range(3):
        (dims,) = take()
        n_seq, rows, H, dk, dv = (int(x) for x in dims)
        (lens,) = take()
        q, k, v, beta, la = take(5)
        s0, d_o, d_sT = take(3)
        o, mag, s1, dq, dkk, dvv, db, dla, ds0 = take(9)
        q, k, la = (x.reshape(rows, H, dk) for x in (q, k, la))
        v = v.reshape(rows, H, dv)
        beta = beta.reshape(rows, H)
        row0 = np.concatenate([[0], np.cumsum(lens)[:-1]]).astype(np.int64)
        init = s0.reshape(n_seq, H, dk, dv) if s0.size else None
        ro, rs1, rmag = oracle.run_rows(q, k, v, beta, la, row0, lens, 1, init, with_magnitude=True)
        assert np.array_equal(o, np.nan_to_num(ro.ravel(), nan=0.0))
        if mag.size:
            assert np.array_equal(mag, np.nan_to_num(rmag.ravel(), nan=0.0))
        assert np.array_equal(s1, rs1.ravel())
        cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
        ref = oracle.varlen_backward(q[None], k[None], v[None], beta[None], la[None],
                                     d_o.reshape(1, rows, H, dv), cu, init,
                                     d_sT.reshape(n_seq, H, dk, dv))
        for name, got in (("dq", dq), ("dk", dkk), ("dv", dvv), ("dbeta", db),
                          ("dlog_alpha", dla), ("dinitial_state", ds0)):
            assert np.array_equal(got, np.asarray(ref[name]).ravel()), name
    (dims,) = take()
    rows, H, dk = (int(x) for x in dims)
    qr, kr, br, ar, q, k, b, la = take(8)
    rq, rk, rb, rla = oracle.prepare(qr.reshape(rows, H, dk), kr.reshape(rows, H, dk),
                                     br.reshape(rows, H), ar.reshape(rows, H, dk))
    for got, want in ((q, rq), (k, rk), (b, rb), (la, rla)):
        assert np.array_equal(got, np.asarray(want).ravel())
    assert pos == len(recs)


@pytest.mark.skipif(shutil.which("g++") is None or not os.path.exists("/opt/rocm/lib/libamdhip64.so"),
                    reason="g++ and the HIP runtime are needed")
def test_c_abi_host_code_under_sanitizers(tmp_path):
    from gated_delta_rule_113_amd import build
    objs = sorted(glob.glob(os.path.join(build.BUILD_DIR, "*.hip.o")))
    srcs = sorted(glob.glob(os.path.join(CSRC, "*.hip")))
    if len(objs) != len(srcs) or any(os.path.getmtime(o) < os.path.getmtime(s)
                                     for o, s in zip(objs, sorted(srcs))):
        build.build()
        objs = sorted(glob.glob(os.path.join(build.BUILD_DIR, "*.hip.o")))
    flags = ["-O1", "-g", "-std=c++17", "-D__HIP_PLATFORM_AMD__", "-I", "/opt/rocm/include",
             "-I", os.path.join(ROOT, "include"), "-I", CSRC] + SAN
    host = []
    for src in [os.path.join(CSRC, f) for f in ("kda_api.cpp", "kda_runtime.cpp", "kda_plan.cpp")] + \
            [os.path.join(HERE, "abi_driver.cpp")]:
        obj = str(tmp_path / (os.path.basename(src) + ".o"))
        _run(["g++"] + flags + ["-c", src, "-o", obj])
        host.append(obj)
    exe = str(tmp_path / "abi_driver")
    _run(["g++"] + SAN + ["-o", exe] + host + objs +
         ["-L/opt/rocm/lib", "-lamdhip64", "-Wl,-rpath,/opt/rocm/lib"])
    r = _run([exe], env=ENV)
    assert "0 failure(s)" in r.stdout
