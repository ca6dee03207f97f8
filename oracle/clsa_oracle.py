"""Plain fp64 CPU oracle of one CLSA decode / prefill step.

TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the benchmark's
CPU-baseline leg may import this module.  The product path (the HIP library and
its Python binding) never calls it, and it shares no code with that path: the
only common dependency is the seeded input generator ``clsa_synth``, which holds
none of the method's arithmetic.

Sources (page titles as published; sections named on the page):

* [SUM] picx.dev summary of "You Only Index Once: Cross-Layer Sparse Attention
  with Shared Routing", section Methodology > Architecture Overview:
  eq. 1 (index projections from the shared hidden states, ``index_projection``), eq. 2 (routing
  scores ``I = Q_idx K_idx^T`` and ``S_t = TopK(I_t, k)``, computed once) and
  eq. 3 (every cross-decoder layer l attends with its own query ``Q_t^(l)`` to
  the selected rows ``K_{S_t}, V_{S_t}`` of the one shared cache); section
  Multi-Layer Distillation, eq. 4-5 (``distill_target``, ``distill_kl``).
* [FORUM] zhichai.net explainer "You Only Index Once ... (CLSA) Explained",
  section Background: Attention and Its Limits (softmax(Q K^T / sqrt(d_k)) V),
  and section CLSA: Sharing the Index Across Layers (the Selector gathers KV
  rows by the shared index).

Readings taken where the pages leave a step open:

* scores: plain dot product, no scale, no activation, single head;
* decode row b sees all N_b cached tokens; prefill row t sees tokens 0..t;
* |S_t| = min(k, visible tokens); ties at the k-th score go to the lower index;
  S_t is returned in ascending index order;
* one S_t per query row, shared by every layer and every head;
* attention scale 1/sqrt(head_dim); query head h reads KV head floor(h*Hkv/Hq).

Everything is float64.  Parity: scores, selection and attention are pinned by
the CPU tests in ``tests/test_oracle_pins.py`` (closed forms, brute force on
tiny inputs, special cases reducing to a library attention routine).
"""
from __future__ import annotations

import numpy as np


# ---------------------------------------------------------------------------------------------
# eq. 1: indexer queries and keys projected from the shared hidden states ([SUM] Architecture
# Overview: Q_idx = H W_idx^Q, K_idx = H W_idx^K)
# ---------------------------------------------------------------------------------------------
def index_projection(h_rows: np.ndarray, w_rows: np.ndarray) -> np.ndarray:
    """One projection of eq. 1 for the given hidden-state rows.

    h_rows: (n, d_model) float64.  w_rows: (d_idx, d_model) float64, row j holding the weights
    of indexer channel j (the projection matrix transposed).  Returns (n, d_idx) float64 with
    out[t, j] = sum_c h[t, c] * w[j, c].
    """
    h = np.asarray(h_rows, dtype=np.float64)
    w = np.asarray(w_rows, dtype=np.float64)
    assert h.ndim == 2 and w.ndim == 2 and h.shape[1] == w.shape[1]
    return h @ w.T


def round_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float64 values to the nearest bf16 value, ties to even; uint16 bit patterns.

    bf16 keeps 8 significant bits: writing x = f * 2**e with 1/2 <= |f| < 1, the result is
    round(f * 2**8) * 2**(e - 8) with halves going to the even integer.  For finite values in
    the normal range (the only ones the path produces)."""
    x = np.asarray(x, dtype=np.float64)
    out = np.zeros(x.shape, dtype=np.float64)
    nz = x != 0
    _, e = np.frexp(x[nz])
    quantum = np.ldexp(1.0, e - 8)
    out[nz] = np.round(x[nz] / quantum) * quantum   # np.round rounds halves to even
    f32 = out.astype(np.float32)
    assert np.all(f32.astype(np.float64) == out), "bf16 value outside the fp32 range"
    return (f32.view(np.uint32) >> np.uint32(16)).astype(np.uint16)


# ---------------------------------------------------------------------------------------------
# eq. 2, first half: routing scores  I_t[j] = q_idx,t . K_idx[j]      ([SUM] Architecture Overview)
# ---------------------------------------------------------------------------------------------
def index_scores(q_idx_row: np.ndarray, k_idx_rows: np.ndarray) -> np.ndarray:
    """Score of every visible token for one query row.

    q_idx_row: (d_idx,) float64; k_idx_rows: (n, d_idx) float64 (the n visible tokens,
    in cache order).  Returns (n,) float64: the plain dot products (no scale).
    """
    q = np.asarray(q_idx_row, dtype=np.float64)
    k = np.asarray(k_idx_rows, dtype=np.float64)
    assert k.ndim == 2 and q.shape == (k.shape[1],)
    return k @ q


def assert_scores_exact(scores: np.ndarray, unit: float) -> None:
    """Precondition of the bit-exact comparison: every score is an integer multiple of
    ``unit`` with magnitude below 2**24 units, so fp32 accumulation in any order is exact."""
    s = np.asarray(scores, dtype=np.float64) / unit
    assert np.all(s == np.round(s)), "score not a multiple of the exactness unit"
    assert np.all(np.abs(s) < 2.0 ** 24), "score too large for exact fp32 accumulation"


# ---------------------------------------------------------------------------------------------
# eq. 2, second half: S_t = TopK(I_t, k), token level, once per step   ([SUM] Architecture Overview)
# ---------------------------------------------------------------------------------------------
def topk_select(scores: np.ndarray, k: int) -> np.ndarray:
    """The selected token set of one row.

    Order tokens by (score descending, index ascending), keep the first min(k, n) and
    return them as ascending int64 indices.  -0.0 and +0.0 compare equal (numeric order).
    """
    s = np.asarray(scores, dtype=np.float64)
    n = s.shape[0]
    if k < 1:
        raise ValueError("k must be >= 1")
    m = min(k, n)
    order = np.lexsort((np.arange(n), -s))   # last key is primary: -score ascending, then index
    return np.sort(order[:m]).astype(np.int64)


def pad_selection(sel: np.ndarray, k: int) -> tuple:
    """(idx[k] int32 with -1 padding, count) - the canonical layout of one selected row."""
    out = np.full(k, -1, dtype=np.int32)
    out[: len(sel)] = sel
    return out, len(sel)


# ---------------------------------------------------------------------------------------------
# eq. 3 with the attention of [FORUM] Background: O^(l) = softmax(Q^(l) K_S^T / sqrt(d)) V_S
# ---------------------------------------------------------------------------------------------
def sparse_attention(q: np.ndarray, k_sel: np.ndarray, v_sel: np.ndarray, scale: float | None = None) -> np.ndarray:
    """Attention of one query row over its selected rows, for every layer and head.

    q: (Lc, Hq, hd) float64 - the row's per-layer queries.
    k_sel, v_sel: (m, Hkv, hd) float64 - the m selected rows of the shared cache
    (the same rows for every layer and head).  Query head h reads KV head h // (Hq // Hkv).
    Returns (Lc, Hq, hd) float64.
    """
    q = np.asarray(q, dtype=np.float64)
    k_sel = np.asarray(k_sel, dtype=np.float64)
    v_sel = np.asarray(v_sel, dtype=np.float64)
    lc, hq, hd = q.shape
    m, hkv, hd2 = k_sel.shape
    assert hd2 == hd and v_sel.shape == k_sel.shape and hq % hkv == 0 and m >= 1
    if scale is None:
        scale = 1.0 / np.sqrt(hd)
    group = hq // hkv
    out = np.empty((lc, hq, hd), dtype=np.float64)
    for h in range(hq):
        g = h // group
        logits = (q[:, h, :] @ k_sel[:, g, :].T) * scale          # (Lc, m)
        logits = logits - logits.max(axis=1, keepdims=True)
        p = np.exp(logits)
        out[:, h, :] = (p @ v_sel[:, g, :]) / p.sum(axis=1, keepdims=True)
    return out


# ---------------------------------------------------------------------------------------------
# eq. 4-5: the multi-layer distillation target and loss ([SUM] Methodology, Multi-Layer
# Distillation): the attention distributions of every layer and head, averaged, against the
# indexer's softmax(I_t)
# ---------------------------------------------------------------------------------------------
def distill_target(q: np.ndarray, k_rows: np.ndarray, scale: float | None = None) -> np.ndarray:
    """A-bar_t of eq. 4 for one query position: the mean over every layer l and query head h of
    the attention distribution softmax(q[l, h] . K_g^T * scale) over the position's visible keys,
    with g = h // (Hq // Hkv) and scale 1/sqrt(head_dim) by default.

    q: (L, Hq, hd) float64; k_rows: (n, Hkv, hd) float64.  Returns (n,) float64.
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k_rows, dtype=np.float64)
    lc, hq, hd = q.shape
    n, hkv, hd2 = k.shape
    assert hd2 == hd and hq % hkv == 0 and n >= 1
    if scale is None:
        scale = 1.0 / np.sqrt(hd)
    group = hq // hkv
    total = np.zeros(n, dtype=np.float64)
    for h in range(hq):
        logits = (q[:, h, :] @ k[:, h // group, :].T) * scale     # (L, n)
        logits = logits - logits.max(axis=1, keepdims=True)
        p = np.exp(logits)
        total += (p / p.sum(axis=1, keepdims=True)).sum(axis=0)
    return total / (lc * hq)


def distill_kl(abar: np.ndarray, scores: np.ndarray) -> float:
    """KL(A-bar_t || softmax(I_t)) of eq. 5 for one position, natural log:
    sum_j A_j (log A_j - log softmax(I_t)_j), with 0 log 0 = 0.  The stop-gradient on A-bar
    does not change the value."""
    a = np.asarray(abar, dtype=np.float64)
    s = np.asarray(scores, dtype=np.float64)
    s = s - s.max()
    log_q = s - np.log(np.exp(s).sum())
    nz = a > 0
    return float(np.sum(a[nz] * (np.log(a[nz]) - log_q[nz])))


# ---------------------------------------------------------------------------------------------
# One query row of the step: scores -> TopK once -> gather -> all L layers over the same set
# ---------------------------------------------------------------------------------------------
def step_row(q_idx_row: np.ndarray, k_idx_rows: np.ndarray, q_layers: np.ndarray, fetch_kv, k: int,
             scale: float | None = None) -> dict:
    """The whole hot path for one query row (decode sequence, or prefill position).

    fetch_kv(local_indices) -> (K rows, V rows), each (m, Hkv, hd) float64: the Selector step
    ([FORUM] CLSA: Sharing the Index Across Layers) reading the shared cache by index.
    Returns dict(scores, sel, out) with out (L, Hq, hd).
    """
    scores = index_scores(q_idx_row, k_idx_rows)
    sel = topk_select(scores, k)
    k_sel, v_sel = fetch_kv(sel)
    out = sparse_attention(q_layers, k_sel, v_sel, scale)
    return {"scores": scores, "sel": sel, "out": out}
