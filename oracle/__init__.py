"""CPU fp64 oracle of the CLSA step - test infrastructure only.

Only ``tests/``, ``__graft_entry__.smoke()`` and the benchmark's CPU-baseline leg may
import this package; the product path never does.
"""
from .clsa_oracle import (assert_scores_exact, index_scores, pad_selection, sparse_attention, step_row,
                          topk_select)

__all__ = ["index_scores", "assert_scores_exact", "topk_select", "pad_selection", "sparse_attention", "step_row"]
