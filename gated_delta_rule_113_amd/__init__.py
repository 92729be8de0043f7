"""Kimi Delta Attention (KDA) on AMD Instinct MI355X (gfx950).

The computation lives in ``libkda.so`` (hand-written HIP kernels behind the C
ABI of ``include/kda.h``); this package is its thin Python binding:

    kda_prefill(q, k, v, beta, log_alpha, initial_state=None) -> (o, final_state)
    kda_varlen_prefill(q, k, v, beta, log_alpha, cu_seqlens, initial_state=None)
        -> (o, final_state)
    kda_decode_step(q, k, v, beta, log_alpha, state) -> o      (state in place)
    kda_prefill_raw / kda_varlen_prefill_raw / kda_decode_step_raw
        (the same on raw projections: q, k normalised, beta and log_alpha
        logits, all inside the kernels)
    kda_decode_tokens(q, k, v, beta, log_alpha, state, n_commit=None) -> o
        (K draft tokens from the state; commits an accepted prefix in place)
    kda_decode_step_slots(q, k, v, beta, log_alpha, state_pool, slots) -> o
    kda_varlen_prefill_slots(q, k, v, beta, log_alpha, cu_seqlens, state_pool,
                             init_slots=None, final_slots=None) -> o
        (states in a pool, addressed by int32 slots)
    kda_backward(q, k, v, beta, log_alpha, d_o, initial_state=None,
                 d_final_state=None) -> dict of gradients
    kda_varlen_backward(q, k, v, beta, log_alpha, d_o, cu_seqlens, ...)
        (gradients of a prefill in all its inputs, for training)
    prefill_workspace_size / varlen_prefill_workspace_size /
    backward_workspace_size -> bytes of device workspace a call needs
        (the calls take ``workspace=``: None, "auto" or a caller-owned tensor)

PyTorch is used only for device memory and the current stream.
"""
from ._binding import (  # noqa: F401
    EXPORTS,
    KDA_BF16,
    KDA_F32,
    KDA_PLAN_FULL,
    KDA_PLAN_SEGMENTS,
    KDA_PLAN_UNSEGMENTED,
    KDA_WORKSPACE_AUTO,
    KDAError,
    kda_backward,
    kda_decode_step,
    kda_decode_step_raw,
    kda_decode_step_slots,
    kda_decode_tokens,
    kda_prefill,
    kda_prefill_raw,
    kda_set_prefill_segment,
    kda_varlen_backward,
    kda_varlen_prefill,
    kda_varlen_prefill_raw,
    kda_varlen_prefill_slots,
    backward_workspace_size,
    load_library,
    prefill_workspace_size,
    varlen_prefill_workspace_size,
)

__all__ = ["kda_prefill", "kda_varlen_prefill", "kda_decode_step", "kda_prefill_raw",
           "kda_varlen_prefill_raw", "kda_decode_step_raw", "kda_decode_tokens",
           "kda_decode_step_slots",
           "kda_varlen_prefill_slots", "kda_backward", "kda_varlen_backward",
           "kda_set_prefill_segment", "prefill_workspace_size", "varlen_prefill_workspace_size",
           "backward_workspace_size", "KDA_WORKSPACE_AUTO", "KDA_PLAN_FULL", "KDA_PLAN_SEGMENTS",
           "KDA_PLAN_UNSEGMENTED", "KDAError", "load_library"]
