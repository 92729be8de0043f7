"""Seeded synthetic inputs for the KDA workloads.

This module is the only code shared by the GPU path's tests/benchmark and the
CPU oracle.  It draws random numbers and rounds them to the storage dtypes; it
contains none of the attention arithmetic itself.

Recipe (all draws from numpy PCG64 streams seeded by
``SeedSequence([113, workload_id, tensor_id, ...])``; tensor ids: q=0, k=1,
v=2, beta=3, log_alpha=4, initial state=5, special channels=6, lengths=7,
raw projections=8, loss gradients=9):

* q, k ~ N(0, 1), then L2-normalised per (token, head) in float64;
* v ~ N(0, 1);
* beta = sigmoid(N(0, 1)), one value per (token, head);
* log_alpha = -softplus(N(0, 1)), one value per (token, head, channel);
* "gated" workloads additionally pick, per head, a fixed seeded set of 13 of
  the 128 channels as long-memory channels with log_alpha = -1e-4 * U[0, 1)
  and a disjoint set of 13 fast-forgetting channels with
  log_alpha = -5 - softplus(N(0, 1));
* initial states ~ N(0, 0.02^2) in float32;
* for the backward pass, the loss gradients in the outputs and in the final
  states ~ N(0, 1) in float32 (``loss_gradients``).

Storage: ``dtype="f32"`` keeps every tensor float32; ``dtype="bf16"`` rounds
q, k, v and beta to bfloat16 (round-to-nearest-even from float32) and keeps
log_alpha, states and outputs float32.  The oracle receives the exact float32
widening of the same bits.
"""
from __future__ import annotations

import concurrent.futures
import dataclasses
import math
import os

import numpy as np

ROOT_SEED = 113
Q, K, V, BETA, LOG_ALPHA, STATE, SPECIAL, LENGTHS, RAW, GRAD = range(10)
N_SPECIAL = 13  # round(0.10 * 128)


# ----------------------------------------------------------------------------
# bfloat16 storage helpers
# ----------------------------------------------------------------------------

def bf16_bits(x) -> np.ndarray:
    """Round to bfloat16 (nearest, ties to even, via float32); return uint16 bits."""
    f = np.ascontiguousarray(np.asarray(x, dtype=np.float32))
    u = f.view(np.uint32)
    u = (u + (np.uint32(0x7FFF) + ((u >> 16) & np.uint32(1)))) >> 16  # finite inputs only
    return u.astype(np.uint16)


def bf16_to_f32(bits) -> np.ndarray:
    """Exact widening of bfloat16 bits (uint16) to float32."""
    b = np.ascontiguousarray(np.asarray(bits, dtype=np.uint16))
    return (b.astype(np.uint32) << 16).view(np.float32)


def _workers() -> int:
    return max(1, min(16, len(os.sched_getaffinity(0))))


def _run_parallel(fn, jobs):
    """Run fn(job) for every job on a thread pool (numpy releases the GIL)."""
    with concurrent.futures.ThreadPoolExecutor(max_workers=_workers()) as ex:
        for _ in ex.map(fn, jobs):
            pass


def _rng(*key) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([ROOT_SEED, *key])))


def _softplus(x):
    return np.logaddexp(0.0, x)


def _sigmoid(x):
    return 1.0 / (1.0 + np.exp(-x))


def _unit_rows(x):
    return x / np.linalg.norm(x, axis=-1, keepdims=True)


# ----------------------------------------------------------------------------
# per-head draws (float64), shape [n_tokens, d] or [n_tokens]
# ----------------------------------------------------------------------------

def special_channels(workload: int, head: int, dk: int = 128):
    """Seeded disjoint (long_memory, fast) channel index sets for one head
    (the same for every sequence of the workload)."""
    perm = _rng(workload, SPECIAL, head).permutation(dk)
    n = min(N_SPECIAL, dk // 2)
    return np.sort(perm[:n]), np.sort(perm[n:2 * n])


def draw_head(workload: int, head: int, n_tokens: int, dk: int = 128, dv: int = 128,
              gated: bool = False, key=()):
    """Draw q, k, v, beta, log_alpha for one head as float64 arrays."""
    key = tuple(key)
    q = _unit_rows(_rng(workload, Q, *key, head).standard_normal((n_tokens, dk)))
    k = _unit_rows(_rng(workload, K, *key, head).standard_normal((n_tokens, dk)))
    v = _rng(workload, V, *key, head).standard_normal((n_tokens, dv))
    beta = _sigmoid(_rng(workload, BETA, *key, head).standard_normal(n_tokens))
    ga = _rng(workload, LOG_ALPHA, *key, head)
    log_alpha = -_softplus(ga.standard_normal((n_tokens, dk)))
    if gated:
        slow, fast = special_channels(workload, head, dk)
        log_alpha[:, slow] = -1e-4 * ga.random((n_tokens, slow.size))
        log_alpha[:, fast] = -5.0 - _softplus(ga.standard_normal((n_tokens, fast.size)))
    return q, k, v, beta, log_alpha


def draw_state(workload: int, shape, key=()) -> np.ndarray:
    return (0.02 * _rng(workload, STATE, *tuple(key)).standard_normal(shape)).astype(np.float32)


def loss_gradients(workload: int, o_shape, n_states: int, H: int, dk: int = 128, dv: int = 128):
    """Seeded gradients of a loss in the outputs (``o_shape``, e.g. [B, T, H,
    dv]) and in the final states ([n_states, H, dk, dv]), N(0, 1) float32."""
    d_o = _rng(workload, GRAD, 0).standard_normal(tuple(o_shape)).astype(np.float32)
    d_s = _rng(workload, GRAD, 1).standard_normal((n_states, H, dk, dv)).astype(np.float32)
    return d_o, d_s


def output_gradients(workload: int, B: int, T: int, H: int, dv: int = 128, heads=None) -> np.ndarray:
    """Seeded N(0, 1) float32 gradients of a loss in the outputs, [B, T, H, dv]
    (or the given heads only), one stream per (sequence, head), drawn in
    parallel: for large workloads, where one stream would be slow."""
    heads = list(range(H)) if heads is None else list(heads)
    d_o = np.empty((B, T, len(heads), dv), np.float32)

    def one(job):
        b, j, h = job
        d_o[b, :, j] = _rng(workload, GRAD, 2, b, h).standard_normal((T, dv), dtype=np.float32)

    _run_parallel(one, [(b, j, h) for b in range(B) for j, h in enumerate(heads)])
    return d_o


# ----------------------------------------------------------------------------
# workloads in the library layout
# ----------------------------------------------------------------------------

@dataclasses.dataclass
class KDAInputs:
    """Host copies of one workload.

    ``q, k, v, beta`` are float32 arrays (dtype "f32") or uint16 bfloat16 bits
    (dtype "bf16"); ``log_alpha`` and ``initial_state`` are float32.
    Layouts: dense q/k/log_alpha [B, T, H, dk], v [B, T, H, dv], beta [B, T, H];
    packed (``cu_seqlens`` set) the same with B = 1; decode chains
    [steps, N, H, *].
    """
    q: np.ndarray
    k: np.ndarray
    v: np.ndarray
    beta: np.ndarray
    log_alpha: np.ndarray
    dtype: str
    initial_state: np.ndarray | None = None
    cu_seqlens: np.ndarray | None = None

    def widened(self):
        """(q, k, v, beta, log_alpha) as exact float32 values for the oracle."""
        if self.dtype == "bf16":
            w = [bf16_to_f32(x) for x in (self.q, self.k, self.v, self.beta)]
        else:
            w = [self.q, self.k, self.v, self.beta]
        return (*w, self.log_alpha)


def _store(x, dtype):
    if dtype == "bf16":
        return bf16_bits(x)
    if dtype == "f32":
        return np.asarray(x, dtype=np.float32)
    raise ValueError(dtype)


def dense_prefill(workload: int, B: int, T: int, H: int, dk: int = 128, dv: int = 128,
                  dtype: str = "bf16", gated: bool = False, initial_state: bool = False,
                  heads=None) -> KDAInputs:
    """Dense [B, T, H, *] prefill inputs; sequence b, head h is drawn from the
    streams keyed (workload, tensor, b, h) so one head can be regenerated alone."""
    heads = list(range(H)) if heads is None else list(heads)
    Hs = len(heads)
    q = np.empty((B, T, Hs, dk), np.float32 if dtype == "f32" else np.uint16)
    k = np.empty_like(q)
    la = np.empty((B, T, Hs, dk), np.float32)
    v = np.empty((B, T, Hs, dv), q.dtype)
    beta = np.empty((B, T, Hs), q.dtype)
    def one(job):
        b, j, h = job
        hq, hk, hv, hb, hla = draw_head(workload, h, T, dk, dv, gated, key=(b,))
        q[b, :, j] = _store(hq, dtype)
        k[b, :, j] = _store(hk, dtype)
        v[b, :, j] = _store(hv, dtype)
        beta[b, :, j] = _store(hb, dtype)
        la[b, :, j] = hla

    _run_parallel(one, [(b, j, h) for b in range(B) for j, h in enumerate(heads)])
    s0 = draw_state(workload, (B, H, dk, dv))[:, heads] if initial_state else None
    return KDAInputs(q, k, v, beta, la, dtype, s0)


def varlen_lengths(workload: int, n_seqs: int, lo: int, hi: int) -> np.ndarray:
    """Lengths floor(exp(U[ln lo, ln hi])), the log-uniform length mix."""
    u = _rng(workload, LENGTHS).random(n_seqs)
    return np.floor(np.exp(math.log(lo) + u * (math.log(hi) - math.log(lo)))).astype(np.int64)


def varlen_prefill(workload: int, lengths, H: int, dk: int = 128, dv: int = 128,
                   dtype: str = "bf16", gated: bool = True, resumed: str = "even") -> KDAInputs:
    """Packed prefill inputs [1, T_total, H, *] with cu_seqlens (int32).

    resumed: "even" -> even-indexed sequences start from N(0, 0.02^2) states and
    odd ones from zeros; "all" / "none" as named.
    """
    lengths = np.asarray(lengths, dtype=np.int64)
    n = lengths.size
    cu = np.zeros(n + 1, np.int64)
    cu[1:] = np.cumsum(lengths)
    Tt = int(cu[-1])
    sdt = np.float32 if dtype == "f32" else np.uint16
    q = np.empty((1, Tt, H, dk), sdt)
    k = np.empty_like(q)
    v = np.empty((1, Tt, H, dv), sdt)
    beta = np.empty((1, Tt, H), sdt)
    la = np.empty((1, Tt, H, dk), np.float32)
    def one(job):
        s, h = job
        a, b = int(cu[s]), int(cu[s + 1])
        hq, hk, hv, hb, hla = draw_head(workload, h, b - a, dk, dv, gated, key=(s,))
        q[0, a:b, h] = _store(hq, dtype)
        k[0, a:b, h] = _store(hk, dtype)
        v[0, a:b, h] = _store(hv, dtype)
        beta[0, a:b, h] = _store(hb, dtype)
        la[0, a:b, h] = hla

    _run_parallel(one, [(s, h) for s in range(n) for h in range(H)])
    s0 = draw_state(workload, (n, H, dk, dv))
    if resumed == "even":
        s0[1::2] = 0.0
    elif resumed == "none":
        s0[:] = 0.0
    elif resumed != "all":
        raise ValueError(resumed)
    return KDAInputs(q, k, v, beta, la, dtype, s0, cu.astype(np.int32))


def varlen_prefill_bulk(workload: int, lengths, H: int, dtype: str = "bf16", gated: bool = True,
                        resumed: str = "even") -> KDAInputs:
    """Packed prefill inputs like ``varlen_prefill`` (same distributions and
    state rule) for batches of thousands of sequences: each head's rows are
    drawn for the whole packed batch from one stream keyed (workload, tensor,
    0, head) and then cut at the sequence boundaries, instead of one stream
    per (sequence, head)."""
    lengths = np.asarray(lengths, dtype=np.int64)
    n = lengths.size
    cu = np.zeros(n + 1, np.int64)
    cu[1:] = np.cumsum(lengths)
    dense = dense_prefill(workload, 1, int(cu[-1]), H, dtype=dtype, gated=gated)
    s0 = draw_state(workload, (n, H, 128, 128))
    if resumed == "even":
        s0[1::2] = 0.0
    elif resumed == "none":
        s0[:] = 0.0
    elif resumed != "all":
        raise ValueError(resumed)
    return KDAInputs(dense.q, dense.k, dense.v, dense.beta, dense.log_alpha, dtype, s0,
                     cu.astype(np.int32))


def decode_steps(workload: int, steps: int, N: int, H: int, dk: int = 128, dv: int = 128,
                 dtype: str = "bf16", first_step: int = 0) -> KDAInputs:
    """Inputs for a chain of single-token decode steps, [steps, N, H, *], plus
    the N(0, 0.02^2) initial states [N, H, dk, dv].  Step s draws all N x H
    token vectors at once from the streams keyed (workload, tensor, s)."""
    sdt = np.float32 if dtype == "f32" else np.uint16
    q = np.empty((steps, N, H, dk), sdt)
    k = np.empty_like(q)
    v = np.empty((steps, N, H, dv), sdt)
    beta = np.empty((steps, N, H), sdt)
    la = np.empty((steps, N, H, dk), np.float32)
    def one(i):
        s = first_step + i
        q[i] = _store(_unit_rows(_rng(workload, Q, s).standard_normal((N, H, dk))), dtype)
        k[i] = _store(_unit_rows(_rng(workload, K, s).standard_normal((N, H, dk))), dtype)
        v[i] = _store(_rng(workload, V, s).standard_normal((N, H, dv)), dtype)
        beta[i] = _store(_sigmoid(_rng(workload, BETA, s).standard_normal((N, H))), dtype)
        la[i] = -_softplus(_rng(workload, LOG_ALPHA, s).standard_normal((N, H, dk)))

    _run_parallel(one, range(steps))
    s0 = draw_state(workload, (N, H, dk, dv))
    return KDAInputs(q, k, v, beta, la, dtype, s0)


# ----------------------------------------------------------------------------
# raw projections (inputs of the *_raw entry points, which prepare them)
# ----------------------------------------------------------------------------

def _raw_arrays(workload: int, lead, H: int, dk: int, dv: int):
    """float64 raw draws of shape lead + (H, *): q_raw, k_raw = N(0,1) times a
    per-(token, head) scale e^{N(0, 0.5^2)}; v = N(0,1); beta logits
    N(0, 1.5^2); gate logits N(0,1), except per head 13 channels at N(-9, 1)
    (softplus ~ 1e-4: long memory) and 13 at N(6, 1) (log alpha ~ -6: fast
    forgetting), the raw counterpart of the gated channel mix."""
    lead = tuple(lead)
    r = lambda t: _rng(workload, RAW, t)
    scale = lambda t: np.exp(0.5 * r(t).standard_normal(lead + (H, 1)))
    q = r(Q).standard_normal(lead + (H, dk)) * scale(10 + Q)
    k = r(K).standard_normal(lead + (H, dk)) * scale(10 + K)
    v = r(V).standard_normal(lead + (H, dv))
    b = 1.5 * r(BETA).standard_normal(lead + (H,))
    a = r(LOG_ALPHA).standard_normal(lead + (H, dk))
    for h in range(H):
        slow, fast = special_channels(workload, h, dk)
        a[..., h, slow] -= 9.0
        a[..., h, fast] += 6.0
    return q, k, v, b, a


def raw_prefill(workload: int, B: int, T: int, H: int, dk: int = 128, dv: int = 128,
                dtype: str = "bf16", initial_state: bool = True) -> KDAInputs:
    """Dense [B, T, H, *] raw projections; ``beta`` holds logits and
    ``log_alpha`` gate logits (fp32)."""
    q, k, v, b, a = _raw_arrays(workload, (B, T), H, dk, dv)
    s0 = draw_state(workload, (B, H, dk, dv)) if initial_state else None
    return KDAInputs(_store(q, dtype), _store(k, dtype), _store(v, dtype), _store(b, dtype),
                     a.astype(np.float32), dtype, s0)


def raw_varlen(workload: int, lengths, H: int, dk: int = 128, dv: int = 128,
               dtype: str = "bf16") -> KDAInputs:
    """Packed [1, T_total, H, *] raw projections with cu_seqlens; even-indexed
    sequences resume from N(0, 0.02^2) states, odd ones from zeros."""
    lengths = np.asarray(lengths, dtype=np.int64)
    cu = np.zeros(lengths.size + 1, np.int64)
    cu[1:] = np.cumsum(lengths)
    q, k, v, b, a = _raw_arrays(workload, (1, int(cu[-1])), H, dk, dv)
    s0 = draw_state(workload, (lengths.size, H, dk, dv))
    s0[1::2] = 0.0
    return KDAInputs(_store(q, dtype), _store(k, dtype), _store(v, dtype), _store(b, dtype),
                     a.astype(np.float32), dtype, s0, cu.astype(np.int32))


def raw_decode(workload: int, steps: int, N: int, H: int, dk: int = 128, dv: int = 128,
               dtype: str = "bf16") -> KDAInputs:
    """[steps, N, H, *] raw projections for a chain of decode steps, plus
    N(0, 0.02^2) initial states."""
    q, k, v, b, a = _raw_arrays(workload, (steps, N), H, dk, dv)
    return KDAInputs(_store(q, dtype), _store(k, dtype), _store(v, dtype), _store(b, dtype),
                     a.astype(np.float32), dtype, draw_state(workload, (N, H, dk, dv)))


# ----------------------------------------------------------------------------
# the named workloads (full sizes); tests shrink them through the arguments
# ----------------------------------------------------------------------------

def workload_single(T: int = 256) -> KDAInputs:
    """B=1, H=1, T=256, d=128, everything float32, zero initial state."""
    return dense_prefill(0, 1, T, 1, dtype="f32")


def workload_decode(steps: int = 1024, N: int = 64, H: int = 32) -> KDAInputs:
    """B=64 sequences x H=32 heads, 1024 single-token steps, bf16 q/k/v/beta."""
    return decode_steps(1, steps, N, H)


def workload_chunked(T: int = 32768, H: int = 32, heads=None) -> KDAInputs:
    """B=1, H=32, T=32768, bf16 q/k/v/beta, gated channel mix, zero initial state."""
    return dense_prefill(2, 1, T, H, gated=True, heads=heads)


def workload_million(T: int = 1 << 20, H: int = 32, heads=None) -> KDAInputs:
    """B=1, H=32, T=1,048,576, as the chunked workload (draw a few heads at a time)."""
    return dense_prefill(3, 1, T, H, gated=True, heads=heads)


def workload_varlen(n_seqs: int = 16, H: int = 32, lo: int = 1024, hi: int = 65536) -> KDAInputs:
    """16 packed sequences, lengths log-uniform in [1024, 65536], half resumed."""
    return varlen_prefill(4, varlen_lengths(4, n_seqs, lo, hi), H)


BACKWARD_WORKLOAD = 5
BACKWARD_SHAPE = (8, 4096, 32)  # B, T, H


def workload_backward(B: int = 8, T: int = 4096, H: int = 32, heads=None) -> KDAInputs:
    """Training shape for the backward pass: B=8 sequences of T=4096 tokens,
    H=32, bf16 q/k/v/beta, gated channel mix, zero initial state; its loss
    gradients come from ``loss_gradients(BACKWARD_WORKLOAD, ...)``."""
    return dense_prefill(BACKWARD_WORKLOAD, B, T, H, gated=True, heads=heads)
