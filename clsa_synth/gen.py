"""Seeded, counter-based synthetic inputs for the CLSA decode / prefill step.

This module is shared by the CPU oracle and the GPU path as the ONE source of
input values.  It holds none of the method's arithmetic: it only turns
(seed, tensor id, flat element index) into bf16 bit patterns, plus a few
host-side integer draws (needle positions, ragged sequence lengths).

Generator definition (the device filler in ``synth.hip`` implements exactly
the same steps; a GPU test compares sampled elements bit for bit):

* ``mix(z)`` is the SplitMix64 output function (Steele, Lea & Flood, "Fast
  splittable pseudorandom number generators", OOPSLA 2014): add the golden
  gamma 0x9E3779B97F4A7C15, then xor-shift 30 / multiply 0xBF58476D1CE4E5B9,
  xor-shift 27 / multiply 0x94D049BB133111EB, xor-shift 31.  All arithmetic
  is modulo 2**64.
* The key of a tensor is ``mix(mix(seed) ^ tensor_id)``.
* Draw ``j`` (0..3) of element ``i`` is ``mix(key + 4*i + j)``.
* Uniform integer in ``[lo, hi]``: ``lo + ((draw0 >> 32) * (hi - lo + 1)) >> 32``,
  divided by ``den`` (a power of two) - exact in fp32 and bf16 for the ranges
  used here.
* Approximately N(0, 1) (Irwin-Hall with 12 terms): the twelve 16-bit fields
  of draws 0, 1, 2 are summed as integers; ``z = (sum - 393210) / 65536`` is
  exact in fp32 (|sum - 393210| < 2**24, the divisor a power of two).
* fp32 -> bf16 is round-to-nearest-even on the bit pattern:
  ``(u + 0x7FFF + ((u >> 16) & 1)) >> 16`` (no NaN / Inf can occur).
"""
from __future__ import annotations

import math

import numpy as np

GAMMA = np.uint64(0x9E3779B97F4A7C15)
MUL1 = np.uint64(0xBF58476D1CE4E5B9)
MUL2 = np.uint64(0x94D049BB133111EB)

# Tensor ids: fixed per logical tensor so that every tensor has its own stream.
TID_Q_IDX = 1
TID_K_IDX = 2
TID_Q = 3
TID_K = 4
TID_V = 5
TID_NEEDLE = 6
TID_LEN = 7
TID_Q_IDX_LAYER = 8     # per-layer indexer queries of the routing ablation
TID_H_NEW = 9           # hidden state of each sequence's new token (indexer projection inputs)
TID_W_Q_IDX = 10        # indexer query projection, stored [d_idx, d_model]
TID_W_K_IDX = 11        # indexer key projection, stored [d_idx, d_model]
TID_K_NEW = 12          # K row of each sequence's new token, appended to the cache
TID_V_NEW = 13          # V row of each sequence's new token

KIND_UNIFORM_INT = 0
KIND_NORMAL = 1


def _u64(x) -> np.ndarray:
    return np.asarray(x, dtype=np.uint64)


def mix(z) -> np.ndarray:
    """SplitMix64 output function of ``z`` (uint64 array), modulo 2**64."""
    z = _u64(z) + GAMMA
    z = (z ^ (z >> np.uint64(30))) * MUL1
    z = (z ^ (z >> np.uint64(27))) * MUL2
    return z ^ (z >> np.uint64(31))


def tensor_key(seed: int, tensor_id: int) -> np.uint64:
    with np.errstate(over="ignore"):
        k = mix(mix(_u64(seed & 0xFFFFFFFFFFFFFFFF)) ^ _u64(tensor_id))
    return np.uint64(k)


def draws(key: np.uint64, flat_index: np.ndarray, j: int) -> np.ndarray:
    """Draw ``j`` (0..3) for each element in ``flat_index``."""
    ctr = _u64(flat_index) * np.uint64(4) + np.uint64(j)
    return mix(_u64(key) + ctr)


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round-to-nearest-even fp32 -> bf16, as uint16 bit patterns."""
    u = np.asarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    r = (u + np.uint64(0x7FFF) + ((u >> np.uint64(16)) & np.uint64(1))) >> np.uint64(16)
    return r.astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def bf16_bits_to_f64(b: np.ndarray) -> np.ndarray:
    return bf16_bits_to_f32(b).astype(np.float64)


def uniform_int_bf16(seed: int, tensor_id: int, flat_index, lo: int, hi: int, den: int) -> np.ndarray:
    """bf16 bits of ``randint[lo, hi] / den`` for each flat element index."""
    key = tensor_key(seed, tensor_id)
    with np.errstate(over="ignore"):
        x = draws(key, flat_index, 0)
    m = np.uint64(hi - lo + 1)
    v = ((x >> np.uint64(32)) * m) >> np.uint64(32)
    val = (v.astype(np.int64) + lo).astype(np.float32) / np.float32(den)
    return f32_to_bf16_bits(val)


def normal_bf16(seed: int, tensor_id: int, flat_index) -> np.ndarray:
    """bf16 bits of the 12-term Irwin-Hall approximation of N(0, 1)."""
    key = tensor_key(seed, tensor_id)
    total = np.zeros(np.shape(flat_index), dtype=np.int64)
    with np.errstate(over="ignore"):
        for j in range(3):
            x = draws(key, flat_index, j)
            for f in range(4):
                total += ((x >> np.uint64(16 * f)) & np.uint64(0xFFFF)).astype(np.int64)
    z = (total - 393210).astype(np.float32) / np.float32(65536.0)
    return f32_to_bf16_bits(z)


def needle_positions(seed: int, row: int, n_tokens: int, count: int) -> list[int]:
    """``count`` distinct positions in [0, n_tokens), by rejection, in draw order."""
    if count > n_tokens:
        raise ValueError("more needles than tokens")
    key = tensor_key(seed, TID_NEEDLE)
    out: list[int] = []
    seen: set[int] = set()
    attempt = 0
    with np.errstate(over="ignore"):
        while len(out) < count:
            x = int(mix(_u64(key) + _u64((row << 32) + attempt)))
            attempt += 1
            p = ((x >> 32) * n_tokens) >> 32
            if p not in seen:
                seen.add(p)
                out.append(p)
    return out


def loguniform_lengths(seed: int, batch: int, lo: int, hi: int) -> list[int]:
    """Sequence lengths ``floor(exp(ln lo + u ln(hi/lo)))`` clamped to [lo, hi]."""
    key = tensor_key(seed, TID_LEN)
    out = []
    with np.errstate(over="ignore"):
        for b in range(batch):
            x = int(mix(_u64(key) + _u64(b)))
            u = (x >> 11) * (2.0 ** -53)
            n = int(math.floor(math.exp(math.log(lo) + u * math.log(hi / lo))))
            out.append(min(max(n, lo), hi))
    return out
