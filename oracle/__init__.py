"""CPU float64 oracle of the gated-prefill path (test infrastructure only).

Only the test-suite, the smoke check and the benchmark's CPU-baseline leg may
import this package.  It shares no code with the HIP library.
"""
from .tokengate_oracle import (  # noqa: F401
    causal_attention, gate_score, gated_attention, gated_attention_backward, gated_attention_backward_rows,
    gated_attention_lse, gather_kept,
    gelu, num_kept, random_keys, select_random, select_topk, select_topk_multi, splitmix64,
    rope_inv_freq, rope, qkv_rope, emit_kv,
)
