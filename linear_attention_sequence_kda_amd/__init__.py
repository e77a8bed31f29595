"""MI355X-native KDA / gated delta rule: chunkwise prefill and decode.

The compute path is libkda.so (hand-written HIP for gfx950, C ABI in
``include/kda.h``); this package only marshals arguments to it:

    o, S_final = chunk_fwd(q, k, v, log_alpha, beta, S0)
    o, S_final = chunk_fwd_noalloc(q, k, v, log_alpha, beta, S0)   # no device allocation
    o, S_final = chunk_fwd_varlen(q, k, v, log_alpha, beta, cu_seqlens, max_seqlen, S0)
    o, S_final, z_final = linear_attn_fwd(q, k, v, S0, z0)     # phi = elu + 1
    o          = linear_attn_decode_step(q, k, v, S, z)        # S, z updated in place
    o          = decode_step(q, k, v, log_alpha, beta, S)   # S updated in place
    o          = decode_step_slots(q, k, v, log_alpha, beta, S_pool, slots)
    dq, dk, dv, dlog_alpha, dbeta, dS0 = recurrence_bwd(q, k, v, log_alpha, beta, S0, do, dS_final)
    dq, dk, dv, dlog_alpha, dbeta, dS0 = chunk_bwd(q, k, v, log_alpha, beta, S0, do, dS_final)

Each takes ``flags=NORM_QK | BETA_LOGIT | GATE_RAW`` (any subset) to feed raw
q, k, beta logits and gate pre-activations that the kernels preprocess.

``inputs`` holds the seeded synthetic workloads.
"""

from .binding import (BETA_LOGIT, GATE_RAW, NORM_QK, KdaError, chunk_bwd,  # noqa: F401
                      chunk_bwd_workspace_bytes, chunk_fwd,
                      chunk_fwd_noalloc, chunk_fwd_varlen, chunk_fwd_workspace_bytes, decode_step, linear_attn_decode_step,
                      linear_attn_fwd, decode_step_slots, library, recurrence_bwd,
                      recurrence_bwd_workspace_bytes, timing_enable, timing_read, timing_reset)

__all__ = ["chunk_fwd", "chunk_fwd_noalloc", "chunk_fwd_varlen", "linear_attn_fwd", "linear_attn_decode_step",
           "chunk_fwd_workspace_bytes", "decode_step", "decode_step_slots", "library", "KdaError", "timing_enable", "timing_read", "timing_reset", "NORM_QK",
           "BETA_LOGIT", "GATE_RAW", "chunk_bwd", "chunk_bwd_workspace_bytes", "recurrence_bwd", "recurrence_bwd_workspace_bytes"]
