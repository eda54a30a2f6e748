"""CPU oracle (test infrastructure only; see kvpop_oracle's header)."""
from .kvpop_oracle import (KEY_NONE, KVpopOracle, bf16_to_f64,  # noqa: F401
                           future_attention_target, held_dynamic_by_definition,
                           kept_by_definition, kv_head_of,
                           masked_dense_attention, prefix_thresholds, score_key,
                           softmax_attention)
