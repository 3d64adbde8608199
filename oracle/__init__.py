"""CPU oracle of the DSA hot path (test infrastructure only; see dsa_oracle, warmup_oracle)."""
from .dsa_oracle import (decode_bf16, decode_e4m3fn, dense_causal_attention,  # noqa: F401
                         e4m3fn_value, indexer_scores, row_geometry, run_rows,
                         sparse_attention, token_rows, topk_indices)
from .warmup_oracle import (dense_target, indexer_parts, kl_and_grad,  # noqa: F401
                            row_objective, run_warmup)
