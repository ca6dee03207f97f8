"""CLSA (Cross-Layer Sparse Attention) hot path for MI355X: HIP kernels behind a C ABI.

The compute lives in ``libclsa.so`` (include/clsa.h); ``binding`` marshals arguments to it.
The library is loaded on first use of an entry point (not at package import), so that
``python -m cross_layer_token_amd.build`` works before anything is built.
"""
_EXPORTS = ("HEAD_DIM", "MODE_DECODE", "MODE_PREFILL", "SCHEDULE_LAYER_BATCHED", "SCHEDULE_PER_LAYER",
            "SCHEDULE_PER_LAYER_ROUTING", "CLSAError",
            "distill_kl", "distill_workspace_bytes", "gather_kv", "index_project", "index_scores", "make_dims", "make_rows", "sparse_attn", "step", "step_no_alloc", "topk", "workspace_bytes")

__all__ = ["binding", *_EXPORTS]


def __getattr__(name):
    if name == "binding" or name in _EXPORTS:
        import importlib
        binding = importlib.import_module(__name__ + ".binding")
        return binding if name == "binding" else getattr(binding, name)
    raise AttributeError(f"module {__name__!r} has no attribute {name!r}")
