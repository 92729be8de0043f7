"""Packed prefill of more than 2,000 sequences on the GPU vs the fp64 oracle.

A serving batch packs many short suffixes (restored prefill caches) with a few
long prompts.  With more than 1,024 sequences the planning kernel of the
chunked prefill gives each of its threads several sequences, and its
longest-first ordering and workspace-slot numbering run over thousands of
segments; sequences of at most 16 tokens take the token-by-token kernel in the
same call.  Every output and every final state is checked."""
import numpy as np
import pytest

import gated_delta_rule_113_amd as kda
import kda_inputs as ki
import oracle
from kda_gpu import GroupCheck, device, rel_err_states, rel_err_vectors, upload

CUS = 256          # compute units of an MI355X (the automatic plan's divisor)
MIN_SEGMENT = 1024  # the shortest automatic segment


def many_lengths(seed=60):
    """2,048 lengths in [0, 16], 48 in [17, 1024] and 16 in [1025, 4096],
    shuffled (seeded)."""
    r = np.random.default_rng(seed)
    short = r.integers(0, 17, 2048)
    mid = r.integers(17, 1025, 48)
    long_ = r.integers(1025, 4097, 16)
    lengths = np.concatenate([short, mid, long_])
    return lengths[r.permutation(lengths.size)]


@pytest.fixture
def segment():
    def set_(tokens):
        kda.kda_set_prefill_segment(tokens)
    yield set_
    kda.kda_set_prefill_segment(0)


def test_slot_bound_holds_for_every_candidate_length():
    """Host-side check of the bound the workspace is sized by: only sequences
    cut into two or more segments take slots, and for every candidate
    segment length L >= the shortest one (L_min) their count stays below
    2 * ceil(T_total / L_min)."""
    lengths = many_lengths()
    T_total = int(lengths.sum())
    for H in (2, 8):
        per_cu = -(-T_total * H // CUS)
        seg_max = max(MIN_SEGMENT, -(-per_cu // 64) * 64)
        seg_min = max(MIN_SEGMENT, -(-(seg_max // 8) // 64) * 64)
        bound = 2 * -(-T_total // seg_min)
        L = seg_max
        while L >= seg_min:
            c = -(-lengths // L)
            assert int(c[c > 1].sum()) < bound, (H, L)
            L //= 2
    for L in (64, 128):
        c = -(-lengths // L)
        assert int(c[c > 1].sum()) < 2 * -(-T_total // L), L


@pytest.mark.gpu
@pytest.mark.parametrize("H,seg", [(2, 0), (8, 0), (2, 128)])
def test_many_packed_sequences(segment, H, seg):
    """2,112 packed sequences (2,048 of 0-16 tokens, 48 of 17-1,024, 16 of
    1,025-4,096), even ones resumed from N(0, 0.02^2) states; automatic
    segment lengths (one or three candidates) and forced 128-token segments."""
    torch = __import__("torch")
    lengths = many_lengths()
    inp = ki.varlen_prefill_bulk(61, lengths, H=H)
    assert lengths.size > 2000 and (lengths == 0).any() and lengths.max() > 1024
    segment(seg)
    t = upload(inp, device())
    o, S = kda.kda_varlen_prefill(t["q"], t["k"], t["v"], t["beta"], t["log_alpha"],
                                  t["cu_seqlens"], t["initial_state"])
    torch.cuda.synchronize()
    o, S = o.cpu().numpy(), S.cpu().numpy()
    assert np.all(np.isfinite(o)) and np.all(np.isfinite(S))
    gc = GroupCheck(f"{lengths.size} packed sequences, H={H}, segment {seg or 'automatic'}")
    o_ref, S_ref, mag = gc.timed(oracle.varlen_prefill, *inp.widened(), inp.cu_seqlens,
                                 inp.initial_state, with_magnitude=True)
    # about 8,000 outputs are the first token of a sequence from a zero state,
    # beta (k.q) v, whose read-out can cancel below fp32 resolution (the
    # per-vector measure then uses the read-out's term magnitude; see kda_gpu)
    plain = rel_err_vectors(o[0], o_ref)
    print(f"plain per-vector max rel err {plain:.3e}", flush=True)
    gc.add(rel_err_vectors(o[0], o_ref, mag), rel_err_states(S, S_ref), lengths.size * H)
    empty = np.nonzero(lengths == 0)[0]
    assert np.array_equal(S[empty], inp.initial_state[empty])
    gc.finish()
