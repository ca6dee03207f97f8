"""ctypes binding of the CLSA C ABI (include/clsa.h).

Argument marshalling only: every step of the path runs in ``libclsa.so``.  Device buffers are
passed as torch tensors (or raw integer addresses); the stream defaults to torch's current
stream.  If the library has not been built, importing this module raises ImportError - there is
no fallback implementation.
"""
from __future__ import annotations

import ctypes
import os
from ctypes import POINTER, c_char_p, c_float, c_int32, c_int64, c_size_t, c_void_p

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libclsa.so")

OK, ERR_INVALID_ARGUMENT, ERR_UNSUPPORTED, ERR_WORKSPACE, ERR_DEVICE = 0, 1, 2, 3, 4
MODE_DECODE, MODE_PREFILL = 0, 1
SCHEDULE_LAYER_BATCHED, SCHEDULE_PER_LAYER, SCHEDULE_PER_LAYER_ROUTING = 0, 1, 2
HEAD_DIM = 128

FUNCTIONS = ["clsa_status_string", "clsa_last_error_message", "clsa_abi_version", "clsa_workspace_bytes",
             "clsa_index_scores", "clsa_topk", "clsa_gather_kv", "clsa_sparse_attn", "clsa_step",
             "clsa_index_project", "clsa_distill_workspace_bytes", "clsa_distill_kl", "clsa_step_no_alloc"]
NO_ALLOC_SCRATCH_BYTES = 64 << 20


class Dims(ctypes.Structure):
    _fields_ = [("batch", c_int32), ("d_idx", c_int32), ("topk", c_int32), ("n_layers", c_int32),
                ("hq", c_int32), ("hkv", c_int32), ("head_dim", c_int32), ("sm_scale", c_float)]


class Rows(ctypes.Structure):
    _fields_ = [("mode", c_int32), ("n_rows", c_int32), ("seq", c_int32), ("pos0", c_int32),
                ("max_row_len", c_int32), ("total_tokens", c_int64), ("cu_seqlens_host", POINTER(c_int32))]


class StepArgs(ctypes.Structure):
    _fields_ = [("q_idx", c_void_p), ("k_idx", c_void_p), ("k_cache", c_void_p), ("v_cache", c_void_p),
                ("cu_seqlens", c_void_p), ("q", c_void_p), ("out", c_void_p), ("idx", c_void_p),
                ("count", c_void_p), ("scores", c_void_p), ("ld_scores", c_int64), ("k_sel", c_void_p),
                ("v_sel", c_void_p), ("schedule", c_int32), ("prefill_chunk_rows", c_int32)]


class CLSAError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"{status_string(status)}: {message}")
        self.status = status


def _load(path: str = LIB_PATH):
    # Bind to the HIP runtime torch already carries: libclsa.so needs libamdhip64.so.7 by soname,
    # so loading torch first makes the dynamic linker reuse that runtime instead of pulling a
    # second one (two runtimes in one process cannot share the device or its memory).
    import torch  # noqa: F401
    if not os.path.exists(path):
        raise ImportError(f"{path} is not built; run `python -m cross_layer_token_amd.build`")
    lib = ctypes.CDLL(path)
    P = c_void_p
    sig = {
        "clsa_status_string": (c_char_p, [c_int32]),
        "clsa_last_error_message": (c_char_p, []),
        "clsa_abi_version": (c_int32, []),
        "clsa_workspace_bytes": (c_size_t, [POINTER(Dims), POINTER(Rows), c_int32, c_int32]),
        "clsa_index_scores": (c_int32, [POINTER(Dims), POINTER(Rows), P, P, P, P, c_int64, P]),
        "clsa_topk": (c_int32, [POINTER(Dims), POINTER(Rows), P, P, c_int64, P, P, P, c_size_t, P]),
        "clsa_gather_kv": (c_int32, [POINTER(Dims), POINTER(Rows), P, P, P, P, P, P, P, P]),
        "clsa_sparse_attn": (c_int32, [POINTER(Dims), POINTER(Rows), P, c_int64, c_int32, P, P, P, P, P, P, P, P,
                                       c_int64, P, c_size_t, P]),
        "clsa_step": (c_int32, [POINTER(Dims), POINTER(Rows), POINTER(StepArgs), P, c_size_t, P]),
        "clsa_step_no_alloc": (c_int32, [POINTER(Dims), POINTER(Rows), POINTER(StepArgs), P]),
        "clsa_index_project": (c_int32, [POINTER(Dims), POINTER(Rows), c_int32, P, P, P, P, P, P, P, P, P, P, P]),
        "clsa_distill_workspace_bytes": (c_size_t, [POINTER(Dims), POINTER(Rows)]),
        "clsa_distill_kl": (c_int32, [POINTER(Dims), POINTER(Rows), P, c_int64, P, P, P, c_int64, P, P, P, c_size_t, P]),
    }
    for name, (res, args) in sig.items():
        f = getattr(lib, name)
        f.restype = res
        f.argtypes = args
    return lib


LIB = _load()


def status_string(status: int) -> str:
    return LIB.clsa_status_string(status).decode()


def last_error() -> str:
    return LIB.clsa_last_error_message().decode()


def _ptr(x):
    if x is None:
        return None
    if isinstance(x, int):
        return x
    return x.data_ptr()


def _stream(stream):
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def _check(status: int):
    if status != OK:
        raise CLSAError(status, last_error())


def make_dims(batch, d_idx, topk, n_layers, hq, hkv, head_dim=HEAD_DIM, sm_scale=0.0) -> Dims:
    return Dims(batch, d_idx, topk, n_layers, hq, hkv, head_dim, sm_scale)


def make_rows(mode, n_rows, max_row_len, total_tokens, seq=0, pos0=0, cu_seqlens_host=None) -> Rows:
    r = Rows(mode, n_rows, seq, pos0, max_row_len, total_tokens, None)
    if cu_seqlens_host is not None:
        arr = (c_int32 * len(cu_seqlens_host))(*[int(v) for v in cu_seqlens_host])
        r.cu_seqlens_host = ctypes.cast(arr, POINTER(c_int32))
        r._keep = arr  # keep the host copy alive with the struct
    return r


def workspace_bytes(dims: Dims, rows: Rows, schedule: int = SCHEDULE_LAYER_BATCHED, prefill_chunk_rows: int = 0) -> int:
    n = LIB.clsa_workspace_bytes(ctypes.byref(dims), ctypes.byref(rows), schedule, prefill_chunk_rows)
    if n == 0:
        raise CLSAError(ERR_INVALID_ARGUMENT, last_error())
    return n


def index_scores(dims, rows, q_idx, k_idx, cu_seqlens, scores, ld_scores, stream=None):
    _check(LIB.clsa_index_scores(ctypes.byref(dims), ctypes.byref(rows), _ptr(q_idx), _ptr(k_idx), _ptr(cu_seqlens),
                                 _ptr(scores), ld_scores, _stream(stream)))


def topk(dims, rows, cu_seqlens, scores, ld_scores, idx, count, workspace, workspace_bytes_, stream=None):
    _check(LIB.clsa_topk(ctypes.byref(dims), ctypes.byref(rows), _ptr(cu_seqlens), _ptr(scores), ld_scores, _ptr(idx),
                         _ptr(count), _ptr(workspace), workspace_bytes_, _stream(stream)))


def gather_kv(dims, rows, k_cache, v_cache, cu_seqlens, idx, count, k_sel, v_sel, stream=None):
    _check(LIB.clsa_gather_kv(ctypes.byref(dims), ctypes.byref(rows), _ptr(k_cache), _ptr(v_cache), _ptr(cu_seqlens),
                              _ptr(idx), _ptr(count), _ptr(k_sel), _ptr(v_sel), _stream(stream)))


def index_project(dims, rows, d_model, h, w_q_idx, w_k_idx, cu_seqlens, q_idx, k_idx, k_new=None, v_new=None,
                  k_cache=None, v_cache=None, stream=None):
    _check(LIB.clsa_index_project(ctypes.byref(dims), ctypes.byref(rows), d_model, _ptr(h), _ptr(w_q_idx),
                                  _ptr(w_k_idx), _ptr(cu_seqlens), _ptr(q_idx), _ptr(k_idx), _ptr(k_new), _ptr(v_new),
                                  _ptr(k_cache), _ptr(v_cache), _stream(stream)))


def distill_workspace_bytes(dims: Dims, rows: Rows) -> int:
    n = LIB.clsa_distill_workspace_bytes(ctypes.byref(dims), ctypes.byref(rows))
    if n == 0:
        raise CLSAError(ERR_INVALID_ARGUMENT, last_error())
    return n


def distill_kl(dims, rows, q, q_row_stride, k_cache, cu_seqlens, scores, ld_scores, kl, loss, workspace,
               workspace_bytes_, stream=None):
    _check(LIB.clsa_distill_kl(ctypes.byref(dims), ctypes.byref(rows), _ptr(q), q_row_stride, _ptr(k_cache),
                               _ptr(cu_seqlens), _ptr(scores), ld_scores, _ptr(kl), _ptr(loss), _ptr(workspace),
                               workspace_bytes_, _stream(stream)))


def sparse_attn(dims, rows, q, q_row_stride, n_layers_call, k_sel, v_sel, k_cache, v_cache, cu_seqlens, idx, count,
                out, out_row_stride, workspace, workspace_bytes_, stream=None):
    _check(LIB.clsa_sparse_attn(ctypes.byref(dims), ctypes.byref(rows), _ptr(q), q_row_stride, n_layers_call,
                                _ptr(k_sel), _ptr(v_sel), _ptr(k_cache), _ptr(v_cache), _ptr(cu_seqlens), _ptr(idx),
                                _ptr(count), _ptr(out), out_row_stride, _ptr(workspace), workspace_bytes_,
                                _stream(stream)))


def step(dims, rows, q_idx, k_idx, k_cache, v_cache, cu_seqlens, q, out, idx, count, workspace, workspace_bytes_,
         scores=None, ld_scores=0, k_sel=None, v_sel=None, schedule=SCHEDULE_LAYER_BATCHED, prefill_chunk_rows=0,
         stream=None):
    a = StepArgs(_ptr(q_idx), _ptr(k_idx), _ptr(k_cache), _ptr(v_cache), _ptr(cu_seqlens), _ptr(q), _ptr(out),
                 _ptr(idx), _ptr(count), _ptr(scores), ld_scores, _ptr(k_sel), _ptr(v_sel), schedule,
                 prefill_chunk_rows)
    _check(LIB.clsa_step(ctypes.byref(dims), ctypes.byref(rows), ctypes.byref(a), _ptr(workspace), workspace_bytes_,
                         _stream(stream)))


def step_no_alloc(dims, rows, q_idx, k_idx, k_cache, v_cache, cu_seqlens, q, out, idx, count, scores=None,
                  ld_scores=0, k_sel=None, v_sel=None, schedule=SCHEDULE_LAYER_BATCHED, prefill_chunk_rows=0,
                  stream=None):
    """clsa_step_no_alloc: clsa_step on the library's static per-GPU scratch (no workspace)."""
    a = StepArgs(_ptr(q_idx), _ptr(k_idx), _ptr(k_cache), _ptr(v_cache), _ptr(cu_seqlens), _ptr(q), _ptr(out),
                 _ptr(idx), _ptr(count), _ptr(scores), ld_scores, _ptr(k_sel), _ptr(v_sel), schedule,
                 prefill_chunk_rows)
    _check(LIB.clsa_step_no_alloc(ctypes.byref(dims), ctypes.byref(rows), ctypes.byref(a), _stream(stream)))
