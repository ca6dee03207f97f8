"""A synthetic workload materialised in device memory (torch tensors filled by libclsa_synth.so).

Values are bit-identical to the host generator of ``clsa_synth.gen`` (a GPU test compares
sampled elements).  Needles are planted on the device from the host-computed (token, row) list.
"""
from __future__ import annotations

import ctypes
import os

import numpy as np
import torch

from . import gen
from .workload import Workload

_LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libclsa_synth.so")
_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            raise ImportError(f"{_LIB_PATH} is not built; run `python -m cross_layer_token_amd.build`")
        L = ctypes.CDLL(_LIB_PATH)
        L.synth_fill_uniform_int.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_uint64, ctypes.c_uint32,
                                             ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_void_p]
        L.synth_fill_normal.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_uint64, ctypes.c_uint32,
                                        ctypes.c_void_p]
        L.synth_plant_needles.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int, ctypes.c_int,
                                          ctypes.c_void_p]
        L.synth_tensor_key.argtypes = [ctypes.c_uint64, ctypes.c_uint32]
        L.synth_tensor_key.restype = ctypes.c_uint64
        for f in (L.synth_fill_uniform_int, L.synth_fill_normal, L.synth_plant_needles):
            f.restype = ctypes.c_int
        _lib = L
    return _lib


def _stream():
    return torch.cuda.current_stream().cuda_stream


def fill_uniform_int(t: torch.Tensor, seed: int, tensor_id: int, lo: int, hi: int, den: int):
    e = lib().synth_fill_uniform_int(t.data_ptr(), t.numel(), seed, tensor_id, lo, hi, den, _stream())
    if e:
        raise RuntimeError(f"synth_fill_uniform_int failed ({e})")


def fill_normal(t: torch.Tensor, seed: int, tensor_id: int):
    e = lib().synth_fill_normal(t.data_ptr(), t.numel(), seed, tensor_id, _stream())
    if e:
        raise RuntimeError(f"synth_fill_normal failed ({e})")


class DeviceWorkload:
    """Inputs of one step of ``w`` in device memory.  bf16 tensors hold raw bit patterns (int16)."""

    def __init__(self, w: Workload, device="cuda", with_q=True, with_kv=True):
        self.w = w
        d = torch.device(device)
        R, T = w.n_rows, w.total_tokens
        self.cu_seqlens = torch.from_numpy(w.cu_seqlens).to(d)
        self.q_idx = torch.empty((R, w.d_idx), dtype=torch.int16, device=d)
        self.k_idx = torch.empty((T, w.d_idx), dtype=torch.int16, device=d)
        fill_uniform_int(self.q_idx, w.seed, gen.TID_Q_IDX, w.idx_lo, w.idx_hi, w.idx_den)
        fill_uniform_int(self.k_idx, w.seed, gen.TID_K_IDX, w.idx_lo, w.idx_hi, w.idx_den)
        pairs = w.needle_pairs()
        if pairs:
            pd = torch.tensor(np.asarray(pairs, dtype=np.int64).reshape(-1), device=d)
            e = lib().synth_plant_needles(self.k_idx.data_ptr(), self.q_idx.data_ptr(), pd.data_ptr(), len(pairs),
                                          w.d_idx, _stream())
            if e:
                raise RuntimeError(f"synth_plant_needles failed ({e})")
            self._pairs = pd
        self.q = None
        self.k_cache = self.v_cache = None
        if with_q:
            self.q = torch.empty((R, w.n_layers, w.hq, w.head_dim), dtype=torch.int16, device=d)
            fill_normal(self.q, w.seed, gen.TID_Q)
        if with_kv:
            self.k_cache = torch.empty((T, w.hkv, w.head_dim), dtype=torch.int16, device=d)
            self.v_cache = torch.empty((T, w.hkv, w.head_dim), dtype=torch.int16, device=d)
            fill_normal(self.k_cache, w.seed, gen.TID_K)
            fill_normal(self.v_cache, w.seed, gen.TID_V)
        torch.cuda.synchronize(d)

    def layer_q_idx(self) -> torch.Tensor:
        """[R, L, d_idx] per-layer indexer queries (the routing ablation), filled on first use."""
        if getattr(self, "_layer_q_idx", None) is None:
            w = self.w
            t = torch.empty((w.n_rows, w.n_layers, w.d_idx), dtype=torch.int16, device=self.q_idx.device)
            fill_uniform_int(t, w.seed, gen.TID_Q_IDX_LAYER, w.idx_lo, w.idx_hi, w.idx_den)
            torch.cuda.synchronize(t.device)
            self._layer_q_idx = t
        return self._layer_q_idx

    def projection_inputs(self, d_model: int) -> dict:
        """Inputs of the new-token indexer projections and cache append (decode):
        h [B, d_model], w_q_idx / w_k_idx [d_idx, d_model], k_new / v_new [B, Hkv, hd]."""
        w = self.w
        d = self.q_idx.device
        h = torch.empty((w.batch, d_model), dtype=torch.int16, device=d)
        wq = torch.empty((w.d_idx, d_model), dtype=torch.int16, device=d)
        wk = torch.empty((w.d_idx, d_model), dtype=torch.int16, device=d)
        fill_uniform_int(h, w.seed, gen.TID_H_NEW, *w.PROJ_H)
        fill_uniform_int(wq, w.seed, gen.TID_W_Q_IDX, *w.PROJ_W)
        fill_uniform_int(wk, w.seed, gen.TID_W_K_IDX, *w.PROJ_W)
        k_new = torch.empty((w.batch, w.hkv, w.head_dim), dtype=torch.int16, device=d)
        v_new = torch.empty((w.batch, w.hkv, w.head_dim), dtype=torch.int16, device=d)
        fill_normal(k_new, w.seed, gen.TID_K_NEW)
        fill_normal(v_new, w.seed, gen.TID_V_NEW)
        torch.cuda.synchronize(d)
        return {"h": h, "w_q_idx": wq, "w_k_idx": wk, "k_new": k_new, "v_new": v_new}

    # sizes of the C ABI, as plain keyword dicts
    def dims(self, sm_scale: float = 0.0) -> dict:
        w = self.w
        return dict(batch=w.batch, d_idx=w.d_idx, topk=w.topk, n_layers=w.n_layers, hq=w.hq, hkv=w.hkv,
                    head_dim=w.head_dim, sm_scale=sm_scale)

    def rows(self, row0: int = 0, n_rows: int | None = None, with_host_cu: bool = True) -> dict:
        w = self.w
        cu = w.cu_seqlens.tolist() if with_host_cu else None
        if w.mode == "decode":
            return dict(mode=0, n_rows=w.batch, max_row_len=w.max_row_len, total_tokens=w.total_tokens,
                        cu_seqlens_host=cu)
        n = w.n_rows - row0 if n_rows is None else n_rows
        return dict(mode=1, n_rows=n, max_row_len=row0 + n, total_tokens=w.total_tokens, seq=0, pos0=row0,
                    cu_seqlens_host=cu)
