"""CPU oracle for the TokenGate gated-prefill path.

TEST INFRASTRUCTURE: imported only by the tests, the smoke check and the
benchmark's CPU-baseline leg.  It shares no code with the HIP library.
"""
from .tokengate_ref import (  # noqa: F401
    compact,
    gate_score,
    gate_select_varlen,
    gated_attention,
    gated_attention_gate_form,
    gated_attention_rope,
    gated_attention_rope_backward,
    gated_attention_backward,
    gated_attention_backward_l1,
    kv_cache_prune,
    bf16_round,
    rope,
    rope_inv_freq,
    score_rows,
    seq_rmsnorm,
    temperature_ratio,
    topk_select,
    widen,
)
