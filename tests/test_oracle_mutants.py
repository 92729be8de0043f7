"""Plant plausible mistakes in a copy of the oracle (on the CPU) and require
each one to be caught by at least one pin.  This shows the pins constrain
every step of the recurrence: the decay, the recall, the compare, the
write, the read-out, the gate indexing, the token order and the state hand-off;
and every step of the input preparation: the gate functions, the per-head
normalisation and the bf16 rounding.
"""
import os
import shutil
import subprocess

import pytest

import oracle
import oracle_pins

with open(oracle.SOURCE) as _f:
    _SRC = _f.read()


def _block(src, title):
    start = src.index("        /* " + title)
    ends = [e for e in (src.find("\n\n", start), src.find("\n    }\n", start)) if e >= 0]
    return src[start:min(ends) + 1] + ("\n" if src[min(ends):min(ends) + 2] == "\n\n" else "")


def _move_after(src, title, after_title):
    blk = _block(src, title)
    src = src.replace(blk, "", 1)
    anchor = _block(src, after_title)
    return src.replace(anchor, anchor + blk, 1)


def _move_before(src, title, before_title):
    blk = _block(src, title)
    src = src.replace(blk, "", 1)
    anchor = _block(src, before_title)
    return src.replace(anchor, blk + anchor, 1)


def _replace(old, new):
    def f(src):
        assert old in src, old
        return src.replace(old, new, 1)
    return f


MUTANTS = {
    "no_decay": _replace("a[i] = exp((double)lat[i]);", "a[i] = 1.0;"),
    "decay_sign": _replace("a[i] = exp((double)lat[i]);", "a[i] = exp(-(double)lat[i]);"),
    "compare_sign": _replace("u[j] = bt * ((double)vt[j] - p[j]);", "u[j] = bt * (p[j] - (double)vt[j]);"),
    "beta_dropped": _replace("u[j] = bt * ((double)vt[j] - p[j]);", "u[j] = ((double)vt[j] - p[j]);"),
    "beta_on_v_only": _replace("u[j] = bt * ((double)vt[j] - p[j]);", "u[j] = bt * (double)vt[j] - p[j];"),
    "recall_with_query": _replace("p[j] += S[i * dv + j] * (double)kt[i];", "p[j] += S[i * dv + j] * (double)qt[i];"),
    "write_dropped": _replace("S[i * dv + j] += (double)kt[i] * u[j];", "(void)u;"),
    "write_with_query": _replace("S[i * dv + j] += (double)kt[i] * u[j];", "S[i * dv + j] += (double)qt[i] * u[j];"),
    "readout_with_key": _replace("ot[j] += S[i * dv + j] * (double)qt[i];", "ot[j] += S[i * dv + j] * (double)kt[i];"),
    "magnitude_signed_state": _replace("mt[j] += fabs(S[i * dv + j]) * fabs((double)qt[i]);",
                                       "mt[j] += S[i * dv + j] * fabs((double)qt[i]);"),
    "magnitude_with_key": _replace("mt[j] += fabs(S[i * dv + j]) * fabs((double)qt[i]);",
                                   "mt[j] += fabs(S[i * dv + j]) * fabs((double)kt[i]);"),
    "readout_before_write": lambda s: _move_before(s, "read-out", "correct"),
    "decay_after_write": lambda s: _move_after(s, "decay", "correct"),
    "decay_after_recall": lambda s: _move_after(s, "decay", "recall"),
    "initial_state_ignored": _replace("if (s0) memcpy(", "if (0) memcpy("),
    "tokens_reversed": _replace("const int64_t row = row0[n] + t * row_step;",
                                "const int64_t row = row0[n] + (len[n] - 1 - t) * row_step;"),
    "beta_wrong_head": _replace("bt = (double)beta[row * H + h];", "bt = (double)beta[row * H];"),
    "gate_wrong_head": _replace("log_alpha + (row * H + h) * dk;", "log_alpha + (row * H) * dk;"),
    "sigmoid_sign": _replace("beta[rh] = (float)(1.0 / (1.0 + exp(-(double)b_raw[rh])));",
                             "beta[rh] = (float)(1.0 / (1.0 + exp((double)b_raw[rh])));"),
    "softplus_sign": _replace("log_alpha[rh * dk + i] = (float)(-sp);", "log_alpha[rh * dk + i] = (float)(sp);"),
    "softplus_as_plain_log": _replace("log1p(exp(a));", "log(exp(a) + 1e-3);"),
    "norm_of_half_vector": _replace("for (int64_t i = 0; i < dk; ++i) ss += (double)x[i] * (double)x[i];",
                                    "for (int64_t i = 0; i < dk / 2; ++i) ss += (double)x[i] * (double)x[i];"),
    "no_bf16_rounding": _replace("out[i] = (float)(round ? round_bf16(y) : y);", "out[i] = (float)y;"),
    "bf16_truncated": _replace("return ldexp(nearbyint(ldexp(m, 8)), e - 8);",
                               "return ldexp(trunc(ldexp(m, 8)), e - 8);"),
    "bwd_recall_term_dropped": _replace("                dkt[i] += acc;", "                (void)acc;"),
    "bwd_gate_uses_entering_state": _replace("for (int64_t j = 0; j < dv; ++j) acc += G[i * dv + j] * S[i * dv + j];",
                                             "for (int64_t j = 0; j < dv; ++j) acc += G[i * dv + j] * Sin[i * dv + j];"),
    "bwd_dp_sign": _replace("dp[j] = -bt * du[j];", "dp[j] = bt * du[j];"),
    "bwd_dq_without_write": _replace("acc += (S[i * dv + j] + (double)kt[i] * u[j]) * dot[j];",
                                     "acc += S[i * dv + j] * dot[j];"),
    "bwd_gradient_not_decayed": _replace("for (int64_t j = 0; j < dv; ++j) G[i * dv + j] *= a[i];", ""),
    "gate_off_by_one_token": _replace("const float *lat = log_alpha + (row * H + h) * dk;",
                                      "const float *lat = log_alpha + ((t ? row - row_step : row) * H + h) * dk;"),
}


@pytest.fixture(scope="module")
def workdir(tmp_path_factory):
    d = tmp_path_factory.mktemp("mutants")
    yield d
    shutil.rmtree(d, ignore_errors=True)


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name, workdir):
    src = MUTANTS[name](_SRC)
    assert src != _SRC
    cfile = os.path.join(workdir, name + ".c")
    with open(cfile, "w") as f:
        f.write(src)
    lib = oracle.load(oracle.build(cfile, os.path.join(workdir, name + ".so")))
    caught = []
    for pin in oracle_pins.ALL_PINS:
        try:
            pin(lib=lib)
        except (AssertionError, ValueError, RuntimeError):
            caught.append(pin.__name__)
    assert caught, f"mutant {name} passed every pin"
