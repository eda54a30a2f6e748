"""CPU oracle (test infrastructure only; see kvpop_oracle's header)."""
from .kvpop_oracle import (KVpopOracle, bf16_to_f64, kept_by_definition,  # noqa: F401
                           kv_head_of, masked_dense_attention, softmax_attention)
