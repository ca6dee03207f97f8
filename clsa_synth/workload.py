"""The five synthetic workloads of the CLSA step, and host-side access to their values.

Every value is defined by ``clsa_synth.gen`` from (seed, tensor id, flat index),
so any element of a multi-GiB cache can be regenerated on the host on demand
without materialising the whole tensor.

Tensor layouts (row-major, bf16 unless stated):

* ``q_idx``  ``[R, d_idx]``         indexer query of each query row
* ``k_idx``  ``[T, d_idx]``         indexer key of every cached token
* ``q``      ``[R, L, Hq, hd]``     per-layer attention query of each row
* ``k``/``v`` ``[T, Hkv, hd]``      the one shared KV cache
* ``cu_seqlens`` int32 ``[B + 1]``  token offsets of the sequences in the cache

``R = B`` for decode (row r is sequence r and sees all its tokens) and
``R = n`` for prefill of one sequence (row t sees tokens 0..t).
"""
from __future__ import annotations

from dataclasses import dataclass, field, replace

import numpy as np

from . import gen


@dataclass(frozen=True)
class Workload:
    name: str
    mode: str                 # "decode" or "prefill"
    seq_lens: tuple           # decode: one length per sequence; prefill: (n,)
    d_idx: int
    topk: int
    n_layers: int
    hq: int
    hkv: int
    head_dim: int
    idx_lo: int               # indexer entries are randint[idx_lo, idx_hi] / idx_den
    idx_hi: int
    idx_den: int
    needles: int              # decode: per sequence; prefill: planted against the last row
    seed: int
    description: str = ""
    # decode only: extra needles at chosen places, (sequence, first local position, count) each;
    # they pack a sequence's largest scores into a chosen stretch of tokens
    planted: tuple = ()
    _cache: dict = field(default_factory=dict, compare=False, repr=False)

    # ---- shapes -------------------------------------------------------------------
    @property
    def batch(self) -> int:
        return len(self.seq_lens)

    @property
    def n_rows(self) -> int:
        return self.batch if self.mode == "decode" else self.seq_lens[0]

    @property
    def total_tokens(self) -> int:
        return int(sum(self.seq_lens))

    @property
    def max_row_len(self) -> int:
        return int(max(self.seq_lens))

    @property
    def cu_seqlens(self) -> np.ndarray:
        return np.concatenate([[0], np.cumsum(self.seq_lens)]).astype(np.int32)

    def row_seq(self, r: int) -> int:
        return r if self.mode == "decode" else 0

    def row_len(self, r: int) -> int:
        return self.seq_lens[r] if self.mode == "decode" else r + 1

    def with_seed(self, seed: int) -> "Workload":
        return replace(self, seed=seed, _cache={})

    # ---- needles -------------------------------------------------------------------
    def needle_pairs(self) -> list:
        """(global token of K_idx, q_idx row it copies) for every planted needle."""
        if "needles" in self._cache:
            return self._cache["needles"]
        pairs = []
        cu = self.cu_seqlens
        if self.needles:
            if self.mode == "decode":
                for b, n in enumerate(self.seq_lens):
                    for p in gen.needle_positions(self.seed, b, n, self.needles):
                        pairs.append((int(cu[b]) + p, b))
            else:
                n = self.seq_lens[0]
                for p in gen.needle_positions(self.seed, 0, n, self.needles):
                    pairs.append((p, n - 1))
        if self.planted:
            assert self.mode == "decode", "planted needles are for decode workloads"
            have = {t for t, _ in pairs}
            for b, start, count in self.planted:
                assert 0 <= start and start + count <= self.seq_lens[b]
                for p in range(start, start + count):
                    if int(cu[b]) + p not in have:
                        pairs.append((int(cu[b]) + p, b))
        self._cache["needles"] = pairs
        return pairs

    def needle_positions_of_row(self, r: int) -> list:
        """Local positions of the needles planted for query row r (must be selected)."""
        cu = self.cu_seqlens
        s = self.row_seq(r)
        return [t - int(cu[s]) for t, src in self.needle_pairs() if src == r]

    # ---- host values (bf16 bit patterns) -------------------------------------------
    def q_idx_bits(self, rows) -> np.ndarray:
        rows = np.asarray(rows, dtype=np.int64).reshape(-1)
        flat = rows[:, None] * self.d_idx + np.arange(self.d_idx)[None, :]
        return gen.uniform_int_bf16(self.seed, gen.TID_Q_IDX, flat, self.idx_lo, self.idx_hi, self.idx_den)

    def k_idx_bits(self, tokens) -> np.ndarray:
        tokens = np.asarray(tokens, dtype=np.int64).reshape(-1)
        flat = tokens[:, None] * self.d_idx + np.arange(self.d_idx)[None, :]
        out = gen.uniform_int_bf16(self.seed, gen.TID_K_IDX, flat, self.idx_lo, self.idx_hi, self.idx_den)
        pairs = self.needle_pairs()
        if pairs:
            lut = dict(pairs)
            hit = [i for i, t in enumerate(tokens.tolist()) if t in lut]
            if hit:
                src = [lut[int(tokens[i])] for i in hit]
                qv = gen.bf16_bits_to_f32(self.q_idx_bits(src))
                out[hit] = gen.f32_to_bf16_bits(qv * np.float32(2.0))
        return out

    def q_idx_layer_bits(self, rows, layer: int) -> np.ndarray:
        """Layer `layer`'s own indexer query of each row (the per-layer routing ablation):
        element (r, l, c) of a [R, L, d_idx] tensor, drawn like q_idx from its own stream."""
        rows = np.asarray(rows, dtype=np.int64).reshape(-1)
        flat = (rows[:, None] * self.n_layers + layer) * self.d_idx + np.arange(self.d_idx)[None, :]
        return gen.uniform_int_bf16(self.seed, gen.TID_Q_IDX_LAYER, flat, self.idx_lo, self.idx_hi, self.idx_den)

    def q_bits(self, rows) -> np.ndarray:
        rows = np.asarray(rows, dtype=np.int64).reshape(-1)
        per = self.n_layers * self.hq * self.head_dim
        flat = rows[:, None] * per + np.arange(per)[None, :]
        return gen.normal_bf16(self.seed, gen.TID_Q, flat).reshape(len(rows), self.n_layers, self.hq, self.head_dim)

    def kv_bits(self, tokens, which: str) -> np.ndarray:
        tokens = np.asarray(tokens, dtype=np.int64).reshape(-1)
        per = self.hkv * self.head_dim
        flat = tokens[:, None] * per + np.arange(per)[None, :]
        tid = gen.TID_K if which == "k" else gen.TID_V
        return gen.normal_bf16(self.seed, tid, flat).reshape(len(tokens), self.hkv, self.head_dim)

    # ---- the step before the routing: the new token of each decode sequence ----------
    # Hidden state h [B, d_model] is randint[-1, 1]; the indexer projections W_q_idx, W_k_idx are
    # stored [d_idx, d_model] (row j = the weights of indexer channel j) with entries
    # randint[-1, 1] / 8; the new K and V rows [B, Hkv, hd] are ~N(0, 1).  With integer h and
    # eighths in W every partial sum of a projection is a multiple of 1/8 below d_model / 8, exact
    # in fp32 in any order, so the bf16 results are the rounding of the exact sums on any device.
    PROJ_H = (-1, 1, 1)
    PROJ_W = (-1, 1, 8)

    def new_token(self, b: int) -> int:
        """Cache row (global) of sequence b's new token: its last position."""
        assert self.mode == "decode"
        return int(self.cu_seqlens[b + 1]) - 1

    def h_new_bits(self, rows, d_model: int) -> np.ndarray:
        rows = np.asarray(rows, dtype=np.int64).reshape(-1)
        flat = rows[:, None] * d_model + np.arange(d_model)[None, :]
        lo, hi, den = self.PROJ_H
        return gen.uniform_int_bf16(self.seed, gen.TID_H_NEW, flat, lo, hi, den)

    def w_idx_bits(self, which: str, d_model: int) -> np.ndarray:
        """[d_idx, d_model] weights of the indexer query ("q") or key ("k") projection."""
        flat = np.arange(self.d_idx * d_model, dtype=np.int64).reshape(self.d_idx, d_model)
        tid = gen.TID_W_Q_IDX if which == "q" else gen.TID_W_K_IDX
        lo, hi, den = self.PROJ_W
        return gen.uniform_int_bf16(self.seed, tid, flat, lo, hi, den)

    def kv_new_bits(self, rows, which: str) -> np.ndarray:
        rows = np.asarray(rows, dtype=np.int64).reshape(-1)
        per = self.hkv * self.head_dim
        flat = rows[:, None] * per + np.arange(per)[None, :]
        tid = gen.TID_K_NEW if which == "k" else gen.TID_V_NEW
        return gen.normal_bf16(self.seed, tid, flat).reshape(len(rows), self.hkv, self.head_dim)

    # ---- fp64 views for the oracle ---------------------------------------------------
    def q_idx_f64(self, rows) -> np.ndarray:
        return gen.bf16_bits_to_f64(self.q_idx_bits(rows))

    def q_idx_layer_f64(self, rows, layer: int) -> np.ndarray:
        return gen.bf16_bits_to_f64(self.q_idx_layer_bits(rows, layer))

    def k_idx_f64(self, tokens) -> np.ndarray:
        return gen.bf16_bits_to_f64(self.k_idx_bits(tokens))

    def q_f64(self, rows) -> np.ndarray:
        return gen.bf16_bits_to_f64(self.q_bits(rows))

    def kv_f64(self, tokens) -> tuple:
        return gen.bf16_bits_to_f64(self.kv_bits(tokens, "k")), gen.bf16_bits_to_f64(self.kv_bits(tokens, "v"))


def _decode(name, lens, d_idx, k, L, hq, hkv, lo, hi, den, needles, seed, desc):
    return Workload(name=name, mode="decode", seq_lens=tuple(int(x) for x in lens), d_idx=d_idx, topk=k,
                    n_layers=L, hq=hq, hkv=hkv, head_dim=128, idx_lo=lo, idx_hi=hi, idx_den=den,
                    needles=needles, seed=seed, description=desc)


def config(i: int, seed: int | None = None) -> Workload:
    """The five workloads, with default seed = config number."""
    s = i if seed is None else seed
    if i == 1:
        return _decode("decode_b1_n4k", [4096], 64, 256, 4, 16, 4, -8, 8, 8, 8, s,
                       "decode B=1 N=4096 d_idx=64 k=256 L=4 Hq=16 Hkv=4 hd=128")
    if i == 2:
        return _decode("decode_b8_n32k", [32768] * 8, 128, 2048, 12, 32, 8, -8, 8, 8, 16, s,
                       "decode B=8 N=32768 d_idx=128 k=2048 L=12 Hq=32 Hkv=8 hd=128")
    if i == 3:
        return _decode("decode_b16_n128k", [131072] * 16, 128, 2048, 16, 32, 8, -8, 8, 8, 32, s,
                       "decode B=16 N=131072 d_idx=128 k=2048 L=16 Hq=32 Hkv=8 hd=128")
    if i == 4:
        return Workload(name="prefill_n8k", mode="prefill", seq_lens=(8192,), d_idx=128, topk=2048,
                        n_layers=8, hq=32, hkv=8, head_dim=128, idx_lo=-8, idx_hi=8, idx_den=8,
                        needles=16, seed=s,
                        description="causal chunked prefill B=1 n=8192 d_idx=128 k=2048 L=8 Hq=32 Hkv=8 hd=128")
    if i == 5:
        lens = gen.loguniform_lengths(s, 64, 4096, 131072)
        return _decode("ragged_decode_b64", lens, 128, 2048, 12, 32, 8, -1, 1, 4, 0, s,
                       "ragged decode B=64 N~logU[4096,131072] d_idx=128 k=2048 L=12 Hq=32 Hkv=8 hd=128, "
                       "indexer entries in {-1,0,1}/4")
    raise ValueError(f"no config {i}")


def custom(mode="decode", seq_lens=(300,), d_idx=64, topk=32, n_layers=2, hq=8, hkv=2, idx_lo=-8, idx_hi=8,
           idx_den=8, needles=0, seed=0, name="custom", planted=()) -> Workload:
    """A small workload of the same value distributions, for tests."""
    return Workload(name=name, mode=mode, seq_lens=tuple(int(x) for x in seq_lens), d_idx=d_idx, topk=topk,
                    n_layers=n_layers, hq=hq, hkv=hkv, head_dim=128, idx_lo=idx_lo, idx_hi=idx_hi,
                    idx_den=idx_den, needles=needles, seed=seed, planted=tuple(planted))
