"""CPU oracle (test infrastructure only; see dsa_oracle)."""
from .dsa_oracle import (visible_count, indexer_scores, select_top_k, softmax_attention,
                         gate_blend, forward_row, forward,
                         dense_causal_attention)

__all__ = ["visible_count", "indexer_scores", "select_top_k", "softmax_attention",
           "gate_blend", "forward_row", "forward", "dense_causal_attention"]
