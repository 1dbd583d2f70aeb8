"""CPU oracle (test infrastructure only; see mqa_oracle's header)."""
from .mqa_oracle import *  # noqa: F401,F403
from .mqa_oracle import (quantize_rows, dequantize_rows, bf16_bits_to_f64,
                         default_softmax_scale, decode_visible, prefill_visible,
                         attend, attention_weights, decode_ref, decode_ref_q8, decode_ref_rows,
                         prefill_ref, lse_partial, lse_merge, hybrid_block_ref,
                         kv_bytes_per_token, int8_kv_bytes_per_key,
                         decode_visible_keys, prefill_visible_pairs,
                         paged_rows, paged_gather, paged_scatter, paged_window_resident)
