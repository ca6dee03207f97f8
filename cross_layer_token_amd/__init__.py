"""CLSA (Cross-Layer Sparse Attention) hot path for MI355X: HIP kernels behind a C ABI.

The compute lives in ``libclsa.so`` (include/clsa.h); ``binding`` marshals arguments to it.
"""
from . import binding
from .binding import (HEAD_DIM, MODE_DECODE, MODE_PREFILL, SCHEDULE_LAYER_BATCHED, SCHEDULE_PER_LAYER, CLSAError,
                      gather_kv, index_scores, make_dims, make_rows, sparse_attn, step, topk, workspace_bytes)

__all__ = ["binding", "HEAD_DIM", "MODE_DECODE", "MODE_PREFILL", "SCHEDULE_LAYER_BATCHED", "SCHEDULE_PER_LAYER",
           "CLSAError", "gather_kv", "index_scores", "make_dims", "make_rows", "sparse_attn", "step", "topk",
           "workspace_bytes"]
