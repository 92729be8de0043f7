"""Pins for the KDA oracle: checks against facts the pages and the mathematics
fix, none of which re-types the oracle's own loop.

Every ``pin_*`` takes ``lib`` (``None`` = the real oracle library, or a
ctypes handle to a deliberately broken copy) and raises AssertionError when
the oracle disagrees.  ``test_oracle_pins.py`` runs them on the real oracle;
``test_oracle_mutants.py`` runs them on planted mistakes and requires each
mistake to be caught.

Sources: "Kimi K3 -- the architecture and infrastructure, explained"
(sections "How the delta rule actually works", "Kimi Delta Attention: the
load-bearing choice", "Serving infrastructure: supernodes and the prefill
cache"); "Inside Kimi K3: How Moonshot AI Built the Largest Open-Source Model"
(section "Technical Details").
"""
from __future__ import annotations

import math
from fractions import Fraction

import numpy as np

import oracle


def _rng(seed):
    return np.random.default_rng(seed)


def _rel(a, b):
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    scale = max(np.max(np.abs(b)), 1e-300)
    return float(np.max(np.abs(a - b)) / scale)


def _random_case(seed, B=2, T=7, H=2, dk=5, dv=3, s0=True):
    r = _rng(seed)
    f = np.float32
    q = r.standard_normal((B, T, H, dk)).astype(f)
    k = (r.standard_normal((B, T, H, dk)) / math.sqrt(dk)).astype(f)
    v = r.standard_normal((B, T, H, dv)).astype(f)
    beta = r.uniform(0.05, 0.95, (B, T, H)).astype(f)
    la = (-r.uniform(0.0, 1.5, (B, T, H, dk))).astype(f)
    S0 = r.standard_normal((B, H, dk, dv)) if s0 else None
    return q, k, v, beta, la, S0


# ---------------------------------------------------------------------------
# brute force: products of the per-token transition matrices
# Phi_t = (I - beta_t k_t k_t^T) Diag(alpha_t), so that
# S_t = Phi_t ... Phi_1 S_0 + sum_s Phi_t ... Phi_{s+1} beta_s k_s v_s^T.
# ---------------------------------------------------------------------------

def _bruteforce_unit(q, k, v, beta, alpha, S0, one, zero, matmul, eye):
    T = len(q)
    Phi = [matmul(eye - beta[t] * np.outer(k[t], k[t]), np.diag(alpha[t])) for t in range(T)]
    outs, S = [], None
    for t in range(T):
        # P(a, b) = Phi_b ... Phi_{a} (identity if a > b)
        def prod(a, b):
            P = eye.copy()
            for j in range(a, b + 1):
                P = matmul(Phi[j], P)
            return P
        S = matmul(prod(0, t), S0)
        for s in range(t + 1):
            S = S + matmul(prod(s + 1, t), beta[s] * np.outer(k[s], v[s]))
        outs.append(matmul(S.T, q[t].reshape(-1, 1)).reshape(-1))
    return np.array(outs), S


def pin_bruteforce_numpy(lib=None):
    """T <= 8: fp64 products of the dense per-token transition matrices."""
    q, k, v, beta, la, S0 = _random_case(1, B=2, T=8, H=2, dk=5, dv=3)
    o, S = oracle.prefill(q, k, v, beta, la, S0, lib=lib)
    B, T, H, dk = q.shape
    for b in range(B):
        for h in range(H):
            alpha = np.exp(la[b, :, h].astype(np.float64))
            ob, Sb = _bruteforce_unit(q[b, :, h].astype(np.float64), k[b, :, h].astype(np.float64),
                                      v[b, :, h].astype(np.float64), beta[b, :, h].astype(np.float64),
                                      alpha, S0[b, h], 1.0, 0.0, np.matmul, np.eye(dk))
            assert _rel(o[b, :, h], ob) < 1e-12, ("o", b, h, _rel(o[b, :, h], ob))
            assert _rel(S[b, h], Sb) < 1e-12, ("S", b, h, _rel(S[b, h], Sb))


def pin_readout_magnitude(lib=None):
    """The read-out magnitudes m_t = |S_t|^T |q_t| against the states of the
    brute-force transition-matrix products (T <= 8); and in the identity case
    (alpha = 1, beta = 0) the closed form |S_0|^T |q_t|."""
    q, k, v, beta, la, S0 = _random_case(3, B=2, T=6, H=2, dk=5, dv=3)
    o, S, m = oracle.prefill(q, k, v, beta, la, S0, lib=lib, with_magnitude=True)
    o2, S2 = oracle.prefill(q, k, v, beta, la, S0, lib=lib)
    assert np.array_equal(o, o2) and np.array_equal(S, S2)
    B, T, H, dk = q.shape
    for b in range(B):
        for h in range(H):
            alpha = np.exp(la[b, :, h].astype(np.float64))
            qq, kk, vv, bb = (x[b, :, h].astype(np.float64) for x in (q, k, v, beta))
            for t in range(T):
                _, St = _bruteforce_unit(qq[:t + 1], kk[:t + 1], vv[:t + 1], bb[:t + 1], alpha[:t + 1],
                                         S0[b, h], 1.0, 0.0, np.matmul, np.eye(dk))
                ref = np.abs(St).T @ np.abs(qq[t])
                assert _rel(m[b, t, h], ref) < 1e-12, (b, h, t)
                assert np.all(m[b, t, h] + 1e-12 >= np.abs(o[b, t, h]))
    z = np.zeros_like(beta)
    _, _, m0 = oracle.prefill(q, k, v, z, np.zeros_like(la), S0, lib=lib, with_magnitude=True)
    for b in range(B):
        for h in range(H):
            ref = np.abs(q[b, :, h].astype(np.float64)) @ np.abs(S0[b, h])
            assert _rel(m0[b, :, h], ref) < 1e-13


def _fmat(a):
    return np.array([[Fraction(float(x)) for x in row] for row in a], dtype=object)


def _fmatmul(A, B):
    n, m = A.shape
    m2, p = B.shape
    assert m == m2
    C = np.empty((n, p), dtype=object)
    for i in range(n):
        for j in range(p):
            acc = Fraction(0)
            for l in range(m):
                acc += A[i, l] * B[l, j]
            C[i, j] = acc
    return C


def pin_bruteforce_exact(lib=None):
    """T <= 8 in exact rational arithmetic (d_k = 4, d_v = 3).

    Inputs are dyadic floats; alpha is taken as the exact rational value of
    the fp64 exp of each fp32 log_alpha, the same number the oracle uses, so
    the only difference left is the oracle's own fp64 rounding."""
    r = _rng(2)
    T, dk, dv = 6, 4, 3
    q = (r.integers(-8, 9, (1, T, 1, dk)) / 8).astype(np.float32)
    k = (r.integers(-4, 5, (1, T, 1, dk)) / 8).astype(np.float32)
    v = (r.integers(-16, 17, (1, T, 1, dv)) / 4).astype(np.float32)
    beta = (r.integers(1, 8, (1, T, 1)) / 8).astype(np.float32)
    choices = np.array([0.0, math.log(0.5), math.log(0.75), math.log(1 / 3)], np.float32)
    la = choices[r.integers(0, 4, (1, T, 1, dk))]
    S0 = r.integers(-3, 4, (1, 1, dk, dv)).astype(np.float64) / 2
    o, S = oracle.prefill(q, k, v, beta, la, S0, lib=lib)
    F = lambda x: Fraction(float(x))
    qf = _fmat(q[0, :, 0]); kf = _fmat(k[0, :, 0]); vf = _fmat(v[0, :, 0])
    bf = [F(b) for b in beta[0, :, 0]]
    af = [[Fraction(math.exp(float(x))) for x in row] for row in la[0, :, 0]]
    eye = np.array([[Fraction(int(i == j)) for j in range(dk)] for i in range(dk)], dtype=object)

    def outer(a, b):
        return np.array([[x * y for y in b] for x in a], dtype=object)

    Phi = [_fmatmul(eye - bf[t] * outer(kf[t], kf[t]),
                    np.array([[af[t][i] if i == j else Fraction(0) for j in range(dk)]
                              for i in range(dk)], dtype=object)) for t in range(T)]
    Sx = _fmat(S0[0, 0])
    for t in range(T):
        # exact recurrence written as the transition product, one step at a time
        Sx = _fmatmul(Phi[t], Sx) + bf[t] * outer(kf[t], vf[t])
        ox = _fmatmul(Sx.T, qf[t].reshape(-1, 1)).reshape(-1)
        ref = np.array([float(x) for x in ox])
        assert _rel(o[0, t, 0], ref) < 1e-13, ("o", t, o[0, t, 0], ref)
    refS = np.array([[float(x) for x in row] for row in Sx])
    assert _rel(S[0, 0], refS) < 1e-13, ("S", S[0, 0], refS)


def pin_identity(lib=None):
    """alpha = 1 and beta = 0: nothing is forgotten or written, S_t = S_0."""
    q, k, v, beta, la, S0 = _random_case(3, B=2, T=9, H=3, dk=6, dv=4)
    la[:] = 0.0
    beta[:] = 0.0
    o, S = oracle.prefill(q, k, v, beta, la, S0, lib=lib)
    assert np.array_equal(S, S0), "state changed under alpha=1, beta=0"
    ref = np.einsum("bhij,bthi->bthj", S0, q.astype(np.float64))
    assert _rel(o, ref) < 1e-14


def _unit_dyadic_keys(r, n, dk, nnz=16):
    """Exactly unit-norm keys: nnz entries of +-1/sqrt(nnz) (nnz a power of 4)."""
    assert int(math.isqrt(nnz)) ** 2 == nnz
    keys = np.zeros((n, dk), np.float32)
    for t in range(n):
        idx = r.choice(dk, nnz, replace=False)
        keys[t, idx] = r.choice([-1.0, 1.0], nnz) / math.sqrt(nnz)
    return keys


def pin_erase_then_write(lib=None):
    """beta = 1 and a unit-norm key: the token's recall S_t^T k_t returns v_t
    exactly ("erase then write"), with or without channel-wise decay before it
    (the decay acts on the old state, which the erase removes along k_t)."""
    r = _rng(4)
    B, T, H, dk, dv = 1, 12, 2, 64, 8
    k = np.stack([_unit_dyadic_keys(r, T, dk) for _ in range(H)], axis=1)[None]
    q = k.copy()                        # read the memory back at the key just written
    v = r.standard_normal((B, T, H, dv)).astype(np.float32)
    beta = np.ones((B, T, H), np.float32)
    S0 = r.standard_normal((B, H, dk, dv))
    for decay in (False, True):
        la = (-r.uniform(0, 2, (B, T, H, dk))).astype(np.float32) if decay \
            else np.zeros((B, T, H, dk), np.float32)
        o, _ = oracle.prefill(q, k, v, beta, la, S0, lib=lib)
        assert _rel(o, v) < 1e-12, ("recall != v", decay, _rel(o, v))


def pin_decay_closed_form(lib=None):
    """beta = 0: S_t = Diag(exp(sum_{j<=t} log_alpha_j)) S_0, including very slow
    (log_alpha in [-1e-4, 0]) and fast (log_alpha <= -5) channels."""
    r = _rng(5)
    B, T, H, dk, dv = 2, 40, 2, 12, 5
    la = (-r.uniform(0, 1.5, (B, T, H, dk))).astype(np.float32)
    la[..., :3] = (-1e-4 * r.random((B, T, H, 3))).astype(np.float32)
    la[..., 3:6] = (-5 - r.uniform(0, 3, (B, T, H, 3))).astype(np.float32)
    q = r.standard_normal((B, T, H, dk)).astype(np.float32)
    k = r.standard_normal((B, T, H, dk)).astype(np.float32)
    v = r.standard_normal((B, T, H, dv)).astype(np.float32)
    beta = np.zeros((B, T, H), np.float32)
    S0 = r.standard_normal((B, H, dk, dv))
    o, S = oracle.prefill(q, k, v, beta, la, S0, lib=lib)
    G = np.cumsum(la.astype(np.float64), axis=1)            # [B, T, H, dk]
    St = np.exp(G)[..., None] * S0[:, None]                  # [B, T, H, dk, dv]
    assert _rel(S, St[:, -1]) < 1e-12
    ref = np.einsum("bthij,bthi->bthj", St, q.astype(np.float64))
    # per token, relative to that token's own scale (fast channels shrink fast)
    for t in range(T):
        assert _rel(o[:, t], ref[:, t]) < 1e-12, t


def pin_channel_locality(lib=None):
    """Changing the forgetting factor of one channel touches only that row of
    the state: (a) with beta = 0, by exactly the ratio of the factors;
    (b) with beta > 0 when every key is zero on that channel."""
    r = _rng(6)
    B, T, H, dk, dv = 1, 10, 1, 8, 6
    q = r.standard_normal((B, T, H, dk)).astype(np.float32)
    k = r.standard_normal((B, T, H, dk)).astype(np.float32) / 3
    v = r.standard_normal((B, T, H, dv)).astype(np.float32)
    la = (-r.uniform(0, 1, (B, T, H, dk))).astype(np.float32)
    S0 = r.standard_normal((B, H, dk, dv))
    ch = 3
    # (a)
    beta0 = np.zeros((B, T, H), np.float32)
    _, Sa = oracle.prefill(q, k, v, beta0, la, S0, lib=lib)
    la2 = la.copy()
    la2[0, 4, 0, ch] -= 0.75
    _, Sb = oracle.prefill(q, k, v, beta0, la2, S0, lib=lib)
    others = [i for i in range(dk) if i != ch]
    assert np.array_equal(Sa[0, 0, others], Sb[0, 0, others])
    ratio = math.exp(float(la2[0, 4, 0, ch]) - float(la[0, 4, 0, ch]))
    assert _rel(Sb[0, 0, ch], ratio * Sa[0, 0, ch]) < 1e-13
    # (b)
    k0 = k.copy()
    k0[..., ch] = 0.0
    beta = r.uniform(0.1, 0.9, (B, T, H)).astype(np.float32)
    _, Sc = oracle.prefill(q, k0, v, beta, la, S0, lib=lib)
    la3 = la.copy()
    la3[0, :, 0, ch] = -2.5
    _, Sd = oracle.prefill(q, k0, v, beta, la3, S0, lib=lib)
    assert np.array_equal(Sc[0, 0, others], Sd[0, 0, others])
    assert not np.array_equal(Sc[0, 0, ch], Sd[0, 0, ch])


def pin_page_delta_rule(lib=None):
    """alpha = 1: the delta-rule update as printed, in the page's orientation
    (state M = S^T is d_v x d_k): v_hat = M k, M <- M - beta (M k - v) k^T,
    and the read-out M q."""
    q, k, v, beta, la, S0 = _random_case(7, B=1, T=9, H=2, dk=6, dv=4)
    la[:] = 0.0
    o, S = oracle.prefill(q, k, v, beta, la, S0, lib=lib)
    for h in range(2):
        M = S0[0, h].T.copy()
        for t in range(q.shape[1]):
            kt = k[0, t, h].astype(np.float64)
            vhat = M @ kt
            M = M - float(beta[0, t, h]) * np.outer(vhat - v[0, t, h], kt)
            assert _rel(o[0, t, h], M @ q[0, t, h].astype(np.float64)) < 1e-12
        assert _rel(S[0, h], M.T) < 1e-12


def _hadamard(n):
    Hm = np.array([[1.0]])
    while Hm.shape[0] < n:
        Hm = np.block([[Hm, Hm], [Hm, -Hm]])
    return Hm


def pin_causal_linear_attention(lib=None):
    """alpha = 1, beta = 1, orthonormal keys, zero start: nothing needs erasing,
    so the delta rule reduces to causal (masked) linear attention:
    S_T = K^T V and o = tril(Q K^T) V."""
    r = _rng(8)
    T, dk, dv = 64, 128, 16
    Hd = _hadamard(64) / 8.0                                  # exact orthonormal rows
    perm = r.permutation(64)
    K = np.zeros((T, dk))
    cols = r.choice(dk, 64, replace=False)
    K[:, cols] = Hd[perm]
    Q = r.standard_normal((T, dk))
    V = r.standard_normal((T, dv))
    f = np.float32
    o, S = oracle.prefill(Q.astype(f)[None, :, None], K.astype(f)[None, :, None],
                          V.astype(f)[None, :, None], np.ones((1, T, 1), f),
                          np.zeros((1, T, 1, dk), f), None, lib=lib)
    Qf, Kf, Vf = (x.astype(f).astype(np.float64) for x in (Q, K, V))
    assert _rel(S[0, 0], Kf.T @ Vf) < 1e-12
    assert _rel(o[0, :, 0], np.tril(Qf @ Kf.T) @ Vf) < 1e-12


def pin_scalar_gate(lib=None):
    """A uniform gate alpha_t * 1 (one forget factor per head, the Gated DeltaNet
    case KDA builds on) commutes with the erase, so with c_t = prod_{j<=t} alpha_t:
    o_t = c_t o'_t and S_T = c_T S'_T, where ' is the ungated run fed v_t / c_t."""
    r = _rng(9)
    B, T, H, dk, dv = 1, 12, 1, 6, 4
    q = r.standard_normal((B, T, H, dk)).astype(np.float32)
    k = (r.standard_normal((B, T, H, dk)) / 2).astype(np.float32)
    beta = r.uniform(0.1, 0.9, (B, T, H)).astype(np.float32)
    a = (-r.uniform(0.0, 0.3, (B, T, H))).astype(np.float32)
    la = np.repeat(a[..., None], dk, axis=-1)
    c = np.exp(np.cumsum(a.astype(np.float64), axis=1))       # [B, T, H]
    # choose v'_t exactly representable, and v_t = c_t v'_t (not exactly
    # representable) is avoided by feeding both runs float32 values and
    # comparing with the rescaling applied to the float32 v actually used
    v = r.standard_normal((B, T, H, dv)).astype(np.float32)
    S0 = r.standard_normal((B, H, dk, dv))
    o, S = oracle.prefill(q, k, v, beta, la, S0, lib=lib)
    # ungated run: fp64 inputs v / c are not float32-exact, so run it in the
    # same page form directly (no decay), which pin_page_delta_rule pins
    M = S0[0, 0].T.copy()
    for t in range(T):
        kt = k[0, t, 0].astype(np.float64)
        vt = v[0, t, 0].astype(np.float64) / c[0, t, 0]
        M = M - float(beta[0, t, 0]) * np.outer(M @ kt - vt, kt)
        assert _rel(o[0, t, 0], c[0, t, 0] * (M @ q[0, t, 0].astype(np.float64))) < 1e-11, t
    assert _rel(S[0, 0], c[0, -1, 0] * M.T) < 1e-11


def pin_resume(lib=None):
    """Prefill-cache resume: running tokens [0, T) equals running [0, t) and
    then [t, T) from the stored state -- bit for bit."""
    q, k, v, beta, la, S0 = _random_case(10, B=2, T=11, H=2, dk=5, dv=4)
    o, S = oracle.prefill(q, k, v, beta, la, S0, lib=lib)
    for t in (0, 1, 5, 10, 11):
        o1, S1 = oracle.prefill(q[:, :t], k[:, :t], v[:, :t], beta[:, :t], la[:, :t], S0, lib=lib) \
            if t > 0 else (np.zeros((2, 0, 2, 4)), S0.copy())
        o2, S2 = oracle.prefill(q[:, t:], k[:, t:], v[:, t:], beta[:, t:], la[:, t:], S1, lib=lib) \
            if t < 11 else (np.zeros((2, 0, 2, 4)), S1)
        assert np.array_equal(np.concatenate([o1, o2], axis=1), o), t
        assert np.array_equal(S2, S), t


def pin_linearity(lib=None):
    """For fixed q, k, beta, alpha the outputs and final state are linear in
    (V, S_0) jointly."""
    r = _rng(11)
    q, k, _, beta, la, _ = _random_case(11, B=1, T=10, H=2, dk=6, dv=4)
    v1 = (r.integers(-64, 65, (1, 10, 2, 4)) / 16).astype(np.float32)
    v2 = (r.integers(-64, 65, (1, 10, 2, 4)) / 16).astype(np.float32)
    s1 = r.standard_normal((1, 2, 6, 4))
    s2 = r.standard_normal((1, 2, 6, 4))
    oa, Sa = oracle.prefill(q, k, v1, beta, la, s1, lib=lib)
    ob, Sb = oracle.prefill(q, k, v2, beta, la, s2, lib=lib)
    oc, Sc = oracle.prefill(q, k, v1 + 3 * v2, beta, la, s1 + 3 * s2, lib=lib)
    assert _rel(oc, oa + 3 * ob) < 1e-12
    assert _rel(Sc, Sa + 3 * Sb) < 1e-12


def pin_varlen_and_layouts(lib=None):
    """Packed sequences are independent (packed == one call per sequence, bit for
    bit); an empty sequence returns its initial state; a [steps, N] decode chain
    equals the dense [N, steps] prefill of the same tokens."""
    q, k, v, beta, la, _ = _random_case(12, B=1, T=23, H=2, dk=5, dv=3)
    lens = [7, 0, 1, 15]
    cu = np.concatenate([[0], np.cumsum(lens)])
    S0 = _rng(12).standard_normal((4, 2, 5, 3))
    o, S = oracle.varlen_prefill(q[0], k[0], v[0], beta[0], la[0], cu, S0, lib=lib)
    for n, (a, b) in enumerate(zip(cu[:-1], cu[1:])):
        if b == a:
            assert np.array_equal(S[n], S0[n])
            continue
        on, Sn = oracle.prefill(q[:, a:b], k[:, a:b], v[:, a:b], beta[:, a:b], la[:, a:b],
                                S0[n:n + 1], lib=lib)
        assert np.array_equal(o[a:b], on[0]), n
        assert np.array_equal(S[n], Sn[0]), n
    # decode chain layout
    qd, kd, vd, bd, lad, _ = _random_case(13, B=3, T=6, H=2, dk=5, dv=3)
    Sd0 = _rng(13).standard_normal((3, 2, 5, 3))
    op, Sp = oracle.prefill(qd, kd, vd, bd, lad, Sd0, lib=lib)
    sw = lambda x: np.ascontiguousarray(np.swapaxes(x, 0, 1))
    oc, Sc = oracle.decode_chain(sw(qd), sw(kd), sw(vd), sw(bd), sw(lad), Sd0, lib=lib)
    assert np.array_equal(sw(oc), op)
    assert np.array_equal(Sc, Sp)


# ---------------------------------------------------------------------------
# input preparation from raw projections (oracle.prepare)
# ---------------------------------------------------------------------------

def pin_prepare_gates(lib=None):
    """sigmoid and -softplus at points where they have closed forms:
    sigmoid(0) = 1/2, sigmoid(ln 3) = 3/4, sigmoid(x) + sigmoid(-x) = 1;
    softplus(0) = ln 2, softplus(x) - softplus(-x) = x, softplus(x) ~ x for
    large x and ~ e^x for very negative x."""
    H, dk = 2, 4
    b = np.array([[0.0, math.log(3.0)], [2.5, -2.5]], np.float32)
    a = np.array([0.0, 1.75, -1.75, 40.0, -40.0, 0.5, -0.5, 3.0], np.float32).reshape(1, H, dk)
    a = np.repeat(a, 2, axis=0)
    z = np.ones((2, H, dk), np.float32)
    _, _, beta, la = oracle.prepare(z, z, b, a, lib=lib)
    assert beta[0, 0] == 0.5
    assert abs(beta[0, 1] - 0.75) < 1e-7
    assert abs(float(beta[1, 0]) + float(beta[1, 1]) - 1.0) < 1e-6
    assert 0.92 < beta[1, 0] < 0.93                    # sigmoid(2.5) = 0.924...
    assert abs(la[0, 0, 0] + math.log(2.0)) < 1e-7
    assert abs((float(la[0, 0, 1]) - float(la[0, 0, 2])) - (-1.75)) < 1e-6
    assert abs(la[0, 0, 3] + 40.0) < 1e-5                 # -softplus(40) = -40 - e^-40
    assert abs(la[0, 1, 0] + math.exp(-40.0)) < 1e-24     # -softplus(-40) = -e^-40
    assert np.all(la < 0)


def pin_prepare_unit_vectors(lib=None):
    """Per (token, head) unit vectors: (3, 4, 0, 0) / 5 = (0.6, 0.8), which
    round to the bf16 values 0.6015625 and 0.80078125 (8 significant bits);
    a scaled axis vector gives the axis exactly; the zero vector stays zero;
    heads of very different scale are normalised independently; without
    rounding the norm is 1 to fp32 accuracy."""
    H, dk = 3, 4
    q = np.array([[[3, 4, 0, 0], [0, 0, -250.0, 0], [0, 0, 0, 0]]], np.float32)
    k = np.array([[[1e-3, 0, 0, 0], [1e3, 1e3, 1e3, 1e3], [0, 5, 0, 0]]], np.float32)
    b = np.zeros((1, H), np.float32)
    qq, kk, _, _ = oracle.prepare(q, k, b, np.zeros((1, H, dk), np.float32), lib=lib)
    assert np.array_equal(qq[0, 0], np.array([0.6015625, 0.80078125, 0, 0], np.float32))
    assert np.array_equal(qq[0, 1], np.array([0, 0, -1, 0], np.float32))
    assert np.array_equal(qq[0, 2], np.zeros(dk, np.float32))
    assert np.array_equal(kk[0, 0], np.array([1, 0, 0, 0], np.float32))
    assert np.array_equal(kk[0, 1], np.full(dk, 0.5, np.float32))
    assert np.array_equal(kk[0, 2], np.array([0, 1, 0, 0], np.float32))
    r = _rng(9).standard_normal((5, H, 16)).astype(np.float32) * np.array([1e-3, 1.0, 1e3], np.float32)[:, None]
    qn, _, _, _ = oracle.prepare(r, r, np.zeros((5, H), np.float32), np.zeros((5, H, 16), np.float32),
                                 round_bf16=False, lib=lib)
    assert np.allclose(np.linalg.norm(qn.astype(np.float64), axis=-1), 1.0, atol=1e-6)
    cos = np.sum(qn.astype(np.float64) * r, axis=-1) / np.linalg.norm(r.astype(np.float64), axis=-1)
    assert np.allclose(cos, 1.0, atol=1e-6)



# ---------------------------------------------------------------------------
# gradients (kda_oracle_backward): central differences of the forward oracle,
# and the closed forms of the identity gate
# ---------------------------------------------------------------------------

def _loss(inputs, d_o, d_s, lib):
    # one thread: thousands of tiny calls, and test workers share the cores
    q, k, v, b, la, s0 = inputs
    o, S = oracle.prefill(q, k, v, b, la, s0, n_threads=1, lib=lib)
    return float(np.sum(o * d_o) + np.sum(S * d_s))


def _fd_check(seed, B, T, H, dk, dv, lib):
    q, k, v, b, la, s0 = _random_case(seed, B=B, T=T, H=H, dk=dk, dv=dv)
    la[..., 0] = -np.float32(5.5)      # a fast-forgetting channel
    la[..., -1] = -np.float32(1e-4)    # a long-memory channel
    r = _rng(seed + 1000)
    d_o = r.standard_normal((B, T, H, dv))
    d_s = r.standard_normal((B, H, dk, dv))
    g = oracle.backward(q, k, v, b, la, d_o, s0, d_s, n_threads=1, lib=lib)
    inputs = [q, k, v, b, la, s0]
    names = ["dq", "dk", "dv", "dbeta", "dlog_alpha", "dinitial_state"]
    for slot, name in enumerate(names):
        x = inputs[slot]
        fd = np.zeros(x.shape)
        for idx in np.ndindex(*x.shape):
            h = 2.0 ** -11 if slot < 5 else 2.0 ** -20
            xp, xm = x.copy(), x.copy()
            xp[idx] += h
            xm[idx] -= h
            step = float(xp[idx]) - float(xm[idx])   # exact: fp32 inputs take exact steps
            lp = _loss(inputs[:slot] + [xp] + inputs[slot + 1:], d_o, d_s, lib)
            lm = _loss(inputs[:slot] + [xm] + inputs[slot + 1:], d_o, d_s, lib)
            fd[idx] = (lp - lm) / step
        err = _rel(g[name], fd)
        assert err < 2e-6, (name, err)


def pin_backward_finite_differences(lib=None):
    """Every gradient entry against central differences of the forward oracle's
    loss sum <dO, o> + <dS_T, S_T>: a short case with two sequences and heads,
    and one of 70 tokens, longer than the backward's 64-token checkpoint
    interval.  Gated mix: one fast (log alpha = -5.5) and one slow (-1e-4)
    channel per head."""
    _fd_check(61, B=2, T=5, H=2, dk=4, dv=3, lib=lib)
    _fd_check(62, B=1, T=70, H=1, dk=3, dv=2, lib=lib)


def pin_backward_identity_gate(lib=None):
    """alpha = 1, beta = 0: the state never changes, o_t = S0^T q_t and S_T =
    S0, so dq_t = S0 dO_t, dS0 = dS_T + sum_t q_t dO_t^T, dv = dk = 0; with
    G_t = dS_T + sum_{s >= t} q_s dO_s^T, the write strength gets
    dbeta_t = (v_t - S0^T k_t) . (G_t^T k_t) and the gate
    dlog_alpha_t[i] = sum_j G_t[i, j] S0[i, j]."""
    B, T, H, dk, dv = 1, 6, 1, 5, 4
    q, k, v, _, _, s0 = _random_case(63, B=B, T=T, H=H, dk=dk, dv=dv)
    b = np.zeros((B, T, H), np.float32)
    la = np.zeros((B, T, H, dk), np.float32)
    r = _rng(64)
    d_o = r.standard_normal((B, T, H, dv))
    d_s = r.standard_normal((B, H, dk, dv))
    g = oracle.backward(q, k, v, b, la, d_o, s0, d_s, lib=lib)
    S0 = s0[0, 0]
    qq, kk, vv, dd = (x[0, :, 0].astype(np.float64) for x in (q, k, v, d_o))
    assert _rel(g["dq"][0, :, 0], dd @ S0.T) < 1e-12
    assert _rel(g["dinitial_state"][0, 0], d_s[0, 0] + qq.T @ dd) < 1e-12
    assert np.all(g["dv"] == 0) and np.all(g["dk"] == 0)
    for t in range(T):
        Gt = d_s[0, 0] + qq[t:].T @ dd[t:]
        assert abs(g["dbeta"][0, t, 0] - (vv[t] - S0.T @ kk[t]) @ (Gt.T @ kk[t])) < 1e-12
        assert _rel(g["dlog_alpha"][0, t, 0], np.sum(Gt * S0, axis=1)) < 1e-12

def pin_backward_gate_identity(lib=None):
    """d log alpha by a second route.  With the cumulative log-decay G_t and the
    rescaled state S^_t = exp(-G_t) S_t, the loss depends on G_t only through
    exp(-G_t) k_t (the written key), exp(G_t) k_t (the read key), exp(G_t) q_t
    and the final state exp(G_T) S^_T.  So dL/dG_t = q_t dq_t + k_t (S'_t dp_t)
    - k_t (G_t u_t) elementwise, plus rowsum(dS_T .* S_T) at t = T, and
    d log alpha_t is the sum of dL/dG_s over s >= t.  Here S'_t and u_t come
    from a numpy forward pass, dp_t = -dv_t (dv = beta du, dp = -beta du), and
    G_t u_t = dk_t - S'_t dp_t; the result must equal the oracle's per-token
    sum of G'_t .* S'_t.  The fast (-5.5) and slow (-1e-4) channels are in."""
    B, T, H, dk, dv = 1, 9, 1, 5, 4
    q, k, v, b, la, s0 = _random_case(67, B=B, T=T, H=H, dk=dk, dv=dv)
    la[..., 0] = -5.5
    la[..., 1] = -1e-4
    r = _rng(68)
    d_o = r.standard_normal((B, T, H, dv))
    d_s = r.standard_normal((B, H, dk, dv))
    g = oracle.backward(q, k, v, b, la, d_o, s0, d_s, lib=lib)
    qq, kk, vv, dd = (x[0, :, 0].astype(np.float64) for x in (q, k, v, d_o))
    bb = b[0, :, 0].astype(np.float64)
    aa = np.exp(la[0, :, 0].astype(np.float64))
    S = s0[0, 0].astype(np.float64)
    Sp = []
    for t in range(T):
        S = aa[t][:, None] * S
        Sp.append(S.copy())
        u = bb[t] * (vv[t] - S.T @ kk[t])
        S = S + np.outer(kk[t], u)
    acc = np.sum(d_s[0, 0] * S, axis=1)
    want = np.zeros((T, dk))
    for t in range(T - 1, -1, -1):
        dp = -g["dv"][0, t, 0]
        read = Sp[t] @ dp
        write = g["dk"][0, t, 0] - read
        acc = acc + qq[t] * g["dq"][0, t, 0] + kk[t] * (read - write)
        want[t] = acc
    assert _rel(g["dlog_alpha"][0, :, 0], want) < 1e-11


def pin_backward_packing(lib=None):
    """Sequences are independent: the packed backward equals the dense
    backward of each sequence alone (rows of other sequences untouched), and
    an empty sequence passes its final-state gradient through unchanged."""
    lengths = [3, 0, 5, 1]
    H, dk, dv = 2, 4, 3
    r = _rng(65)
    cu = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int32)
    Tt = int(cu[-1])
    q, k, v, b, la, _ = _random_case(66, B=1, T=Tt, H=H, dk=dk, dv=dv)
    s0 = r.standard_normal((len(lengths), H, dk, dv)).astype(np.float32)
    d_o = r.standard_normal((Tt, H, dv))
    d_s = r.standard_normal((len(lengths), H, dk, dv))
    g = oracle.varlen_backward(q[0], k[0], v[0], b[0], la[0], d_o, cu, s0, d_s, lib=lib)
    for n, L in enumerate(lengths):
        a, z = cu[n], cu[n + 1]
        one = oracle.backward(q[:, a:z], k[:, a:z], v[:, a:z], b[:, a:z], la[:, a:z],
                              d_o[None, a:z], s0[n:n + 1], d_s[n:n + 1], lib=lib)
        for name in ("dq", "dk", "dv", "dbeta", "dlog_alpha"):
            assert np.array_equal(g[name][a:z], one[name][0]), (n, name)
        assert np.array_equal(g["dinitial_state"][n], one["dinitial_state"][0]), n
    assert np.array_equal(g["dinitial_state"][1], d_s[1])


ALL_PINS = [
    pin_bruteforce_numpy, pin_bruteforce_exact, pin_identity, pin_erase_then_write,
    pin_decay_closed_form, pin_channel_locality, pin_page_delta_rule,
    pin_causal_linear_attention, pin_scalar_gate, pin_resume, pin_linearity,
    pin_varlen_and_layouts, pin_prepare_gates, pin_prepare_unit_vectors,
    pin_backward_finite_differences, pin_backward_identity_gate, pin_backward_gate_identity,
    pin_backward_packing, pin_readout_magnitude,
]
