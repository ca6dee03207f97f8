"""ctypes access to the C++ fp64 oracle (oracle/clsa_oracle.cpp) - test infrastructure only.

The C++ oracle regenerates its inputs from the generator definition itself, so it shares no code
with the Python oracle or the Python generator.  This module offers the same primitives as
``oracle.clsa_oracle`` (index_scores, topk_select, sparse_attention) plus whole-row evaluation.
"""
from __future__ import annotations

import ctypes
import os
from ctypes import POINTER, c_double, c_int, c_int32, c_int64, c_uint16, c_uint64

import numpy as np

from .clsa_oracle import assert_scores_exact, pad_selection  # noqa: F401  (same helpers as the numpy oracle)

_LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libclsa_oracle.so")


class Workload(ctypes.Structure):
    _fields_ = [("mode", c_int32), ("batch", c_int32), ("seq_lens", POINTER(c_int64)), ("d_idx", c_int32),
                ("topk", c_int32), ("n_layers", c_int32), ("hq", c_int32), ("hkv", c_int32), ("head_dim", c_int32),
                ("idx_lo", c_int32), ("idx_hi", c_int32), ("idx_den", c_int32), ("needles", c_int32),
                ("seed", c_uint64)]


def _load(path: str = _LIB_PATH):
    if not os.path.exists(path):
        from . import build
        build.build()
    lib = ctypes.CDLL(path)
    dp, ip = POINTER(c_double), POINTER(c_int32)
    lib.clsa_oracle_gen_uniform.restype = c_uint16
    lib.clsa_oracle_gen_uniform.argtypes = [c_uint64, c_uint64, c_uint64, c_int, c_int, c_int]
    lib.clsa_oracle_gen_normal.restype = c_uint16
    lib.clsa_oracle_gen_normal.argtypes = [c_uint64, c_uint64, c_uint64]
    lib.clsa_oracle_gen_needles.restype = c_int
    lib.clsa_oracle_gen_needles.argtypes = [c_uint64, c_int64, c_int64, c_int32, POINTER(c_int64)]
    lib.clsa_oracle_scores.argtypes = [dp, dp, c_int64, c_int32, dp]
    lib.clsa_oracle_topk.argtypes = [dp, c_int64, c_int32, ip, ip]
    lib.clsa_oracle_attention.argtypes = [dp, dp, dp, c_int64, c_int32, c_int32, c_int32, c_int32, c_double, dp]
    lib.clsa_oracle_row.restype = c_int
    lib.clsa_oracle_row.argtypes = [POINTER(Workload), c_int32, ip, ip, dp, dp]
    lib.clsa_oracle_rows.restype = c_int
    lib.clsa_oracle_rows.argtypes = [POINTER(Workload), ip, c_int32, c_int32, ip, ip, dp, POINTER(c_double)]
    lib.clsa_oracle_row_layer_routing.restype = c_int
    lib.clsa_oracle_row_layer_routing.argtypes = [POINTER(Workload), c_int32, ip, ip, dp]
    lib.clsa_oracle_rows_layer_routing.restype = c_int
    lib.clsa_oracle_rows_layer_routing.argtypes = [POINTER(Workload), ip, c_int32, c_int32, ip, ip, dp]
    return lib


LIB = _load()


def _d(a: np.ndarray):
    return a.ctypes.data_as(POINTER(c_double))


def _i(a: np.ndarray):
    return a.ctypes.data_as(POINTER(c_int32))


def index_scores(q_idx_row, k_idx_rows) -> np.ndarray:
    q = np.ascontiguousarray(q_idx_row, dtype=np.float64)
    k = np.ascontiguousarray(k_idx_rows, dtype=np.float64)
    assert k.ndim == 2 and q.shape == (k.shape[1],)
    out = np.empty(k.shape[0], dtype=np.float64)
    LIB.clsa_oracle_scores(_d(q), _d(k), k.shape[0], k.shape[1], _d(out))
    return out


def topk_select(scores, k: int) -> np.ndarray:
    if k < 1:
        raise ValueError("k must be >= 1")
    s = np.ascontiguousarray(scores, dtype=np.float64)
    idx = np.empty(k, dtype=np.int32)
    cnt = np.zeros(1, dtype=np.int32)
    LIB.clsa_oracle_topk(_d(s), s.shape[0], k, _i(idx), _i(cnt))
    return idx[: int(cnt[0])].astype(np.int64)


def sparse_attention(q, k_sel, v_sel, scale: float | None = None) -> np.ndarray:
    q = np.ascontiguousarray(q, dtype=np.float64)
    k = np.ascontiguousarray(k_sel, dtype=np.float64)
    v = np.ascontiguousarray(v_sel, dtype=np.float64)
    lc, hq, hd = q.shape
    m, hkv, hd2 = k.shape
    assert hd2 == hd and v.shape == k.shape and hq % hkv == 0 and m >= 1
    out = np.empty((lc, hq, hd), dtype=np.float64)
    LIB.clsa_oracle_attention(_d(q), _d(k), _d(v), m, lc, hq, hkv, hd, 0.0 if scale is None else float(scale),
                              _d(out))
    return out


def workload_struct(w) -> tuple:
    lens = np.ascontiguousarray(np.asarray(w.seq_lens, dtype=np.int64))
    s = Workload(0 if w.mode == "decode" else 1, w.batch, lens.ctypes.data_as(POINTER(c_int64)), w.d_idx, w.topk,
                 w.n_layers, w.hq, w.hkv, w.head_dim, w.idx_lo, w.idx_hi, w.idx_den, w.needles,
                 w.seed & 0xFFFFFFFFFFFFFFFF)
    return s, lens   # keep lens alive with the struct


def oracle_row(w, r: int, with_scores: bool = False) -> dict:
    """One row of a workload, inputs regenerated inside the C++ oracle."""
    s, lens = workload_struct(w)
    idx = np.empty(w.topk, dtype=np.int32)
    cnt = np.zeros(1, dtype=np.int32)
    out = np.empty((w.n_layers, w.hq, w.head_dim), dtype=np.float64)
    sc = np.empty(w.row_len(r), dtype=np.float64) if with_scores else None
    rc = LIB.clsa_oracle_row(ctypes.byref(s), r, _i(idx), _i(cnt), _d(out), _d(sc) if with_scores else None)
    assert rc == 0, "clsa_oracle_row rejected its arguments"
    res = {"idx": idx, "count": int(cnt[0]), "out": out}
    if with_scores:
        res["scores"] = sc
    return res


def oracle_rows_timed(w, rows, threads: int) -> tuple:
    """Rows over `threads` host threads (each row single-threaded). Returns (results, seconds)."""
    s, lens = workload_struct(w)
    rows = np.ascontiguousarray(np.asarray(rows, dtype=np.int32))
    n = len(rows)
    idx = np.empty((n, w.topk), dtype=np.int32)
    cnt = np.zeros(n, dtype=np.int32)
    out = np.empty((n, w.n_layers, w.hq, w.head_dim), dtype=np.float64)
    secs = c_double(0.0)
    rc = LIB.clsa_oracle_rows(ctypes.byref(s), _i(rows), n, threads, _i(idx), _i(cnt), _d(out), ctypes.byref(secs))
    assert rc == 0, "clsa_oracle_rows failed"
    return {"idx": idx, "count": cnt, "out": out}, secs.value


def oracle_rows(w, rows, threads: int = 8) -> dict:
    """Several rows over `threads` host threads: idx [n, k], count [n], out [n, L, Hq, hd]."""
    return oracle_rows_timed(w, rows, threads)[0]


def oracle_rows_layer_routing(w, rows, threads: int = 8) -> dict:
    """The per-layer routing ablation (every layer scores with its own indexer query, selects its
    own set and attends over it) for several rows over `threads` host threads:
    idx [n, L, k], count [n, L], out [n, L, Hq, hd]."""
    s, lens = workload_struct(w)
    rows = np.ascontiguousarray(np.asarray(rows, dtype=np.int32))
    n, L = len(rows), w.n_layers
    idx = np.empty((n, L, w.topk), dtype=np.int32)
    cnt = np.zeros((n, L), dtype=np.int32)
    out = np.empty((n, L, w.hq, w.head_dim), dtype=np.float64)
    rc = LIB.clsa_oracle_rows_layer_routing(ctypes.byref(s), _i(rows), n, threads, _i(idx), _i(cnt), _d(out))
    assert rc == 0, "clsa_oracle_rows_layer_routing failed"
    return {"idx": idx, "count": cnt, "out": out}


def oracle_row_layer_routing(w, r: int) -> dict:
    """One row of the per-layer routing ablation: idx [L, k], count [L], out [L, Hq, hd]."""
    s, lens = workload_struct(w)
    L = w.n_layers
    idx = np.empty((L, w.topk), dtype=np.int32)
    cnt = np.zeros(L, dtype=np.int32)
    out = np.empty((L, w.hq, w.head_dim), dtype=np.float64)
    rc = LIB.clsa_oracle_row_layer_routing(ctypes.byref(s), r, _i(idx), _i(cnt), _d(out))
    assert rc == 0, "clsa_oracle_row_layer_routing rejected its arguments"
    return {"idx": idx, "count": cnt, "out": out}


def gen_uniform(seed: int, tid: int, i: int, lo: int, hi: int, den: int) -> int:
    return int(LIB.clsa_oracle_gen_uniform(seed & 0xFFFFFFFFFFFFFFFF, tid, i, lo, hi, den))


def gen_normal(seed: int, tid: int, i: int) -> int:
    return int(LIB.clsa_oracle_gen_normal(seed & 0xFFFFFFFFFFFFFFFF, tid, i))


def gen_needles(seed: int, row: int, n: int, count: int) -> list:
    if count > n:
        raise ValueError("more needles than tokens")
    out = np.empty(count, dtype=np.int64)
    rc = LIB.clsa_oracle_gen_needles(seed & 0xFFFFFFFFFFFFFFFF, row, n, count, out.ctypes.data_as(POINTER(c_int64)))
    assert rc == 0
    return out.tolist()
