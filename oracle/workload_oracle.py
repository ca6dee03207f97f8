"""Oracle results for rows of a synthetic workload (test infrastructure only).

Regenerates, on the host, exactly the inputs a query row needs - its indexer query,
the indexer keys of the tokens it sees, its per-layer queries and only the selected
K/V rows - and runs the fp64 oracle on them.  Inputs come from ``clsa_synth`` alone.
"""
from __future__ import annotations

import numpy as np

from clsa_synth import Workload

from clsa_synth import gen

from .clsa_oracle import (assert_scores_exact, distill_kl, distill_target, index_projection, index_scores,
                          pad_selection, round_bf16_bits, step_row)


def oracle_row(w: Workload, r: int, check_exact: bool = True) -> dict:
    """fp64 oracle of query row r: dict(scores, sel, idx[k], count, out[L, Hq, hd])."""
    cu = w.cu_seqlens
    s = w.row_seq(r)
    n = w.row_len(r)
    base = int(cu[s])
    tokens = base + np.arange(n, dtype=np.int64)

    def fetch(sel):
        return w.kv_f64(base + np.asarray(sel, dtype=np.int64))

    res = step_row(w.q_idx_f64([r])[0], w.k_idx_f64(tokens), w.q_f64([r])[0], fetch, w.topk)
    if check_exact:
        assert_scores_exact(res["scores"], 1.0 / (w.idx_den * w.idx_den))
    res["idx"], res["count"] = pad_selection(res["sel"], w.topk)
    return res


def oracle_rows(w: Workload, rows, keep_scores: bool = False) -> dict:
    """Stack the oracle results of several rows: idx [n, k] int32, count [n], out [n, L, Hq, hd]."""
    idx, cnt, out, scores = [], [], [], []
    for r in rows:
        res = oracle_row(w, int(r))
        idx.append(res["idx"])
        cnt.append(res["count"])
        out.append(res["out"])
        if keep_scores:
            scores.append(res["scores"])
    d = {"idx": np.stack(idx), "count": np.asarray(cnt, dtype=np.int32), "out": np.stack(out)}
    if keep_scores:
        d["scores"] = scores
    return d


def oracle_row_layer_routing(w: Workload, r: int) -> dict:
    """fp64 oracle of query row r under per-layer routing (the ablation without the shared index):
    layer l scores the row's visible tokens with its own indexer query, selects its own set and
    attends with its own query.  dict(idx[L, k], count[L], out[L, Hq, hd])."""
    from .clsa_oracle import index_scores, sparse_attention, topk_select
    cu = w.cu_seqlens
    base = int(cu[w.row_seq(r)])
    tokens = base + np.arange(w.row_len(r), dtype=np.int64)
    k_idx = w.k_idx_f64(tokens)
    q = w.q_f64([r])[0]
    idx, cnt, out = [], [], []
    for l in range(w.n_layers):
        sel = topk_select(index_scores(w.q_idx_layer_f64([r], l)[0], k_idx), w.topk)
        kf, vf = w.kv_f64(base + sel)
        out.append(sparse_attention(q[l:l + 1], kf, vf)[0])
        i, c = pad_selection(sel, w.topk)
        idx.append(i)
        cnt.append(c)
    return {"idx": np.stack(idx), "count": np.asarray(cnt), "out": np.stack(out)}


# ---------------------------------------------------------------------------------------------
# The decode step preceded by the new token's indexer projections (eq. 1) and cache append
# ---------------------------------------------------------------------------------------------
def oracle_projection(w: Workload, d_model: int, rows=None) -> dict:
    """bf16 bits of the new token's indexer query and key for each sequence in `rows` (default:
    all): q_idx [n, d_idx] = RNE(h W_idx^Q), k_idx_new [n, d_idx] = RNE(h W_idx^K)."""
    rows = np.arange(w.batch) if rows is None else np.asarray(rows, dtype=np.int64)
    h = gen.bf16_bits_to_f64(w.h_new_bits(rows, d_model))
    q = index_projection(h, gen.bf16_bits_to_f64(w.w_idx_bits("q", d_model)))
    k = index_projection(h, gen.bf16_bits_to_f64(w.w_idx_bits("k", d_model)))
    return {"q_idx": round_bf16_bits(q), "k_idx_new": round_bf16_bits(k)}


def oracle_row_projected(w: Workload, r: int, d_model: int) -> dict:
    """fp64 oracle of decode row r when the step starts by appending each sequence's new token:
    its indexer query is projected from the hidden state (eq. 1), its indexer key is projected
    into the row's last cache position, and its K/V rows replace that position of the cache.
    dict(scores, sel, idx[k], count, out[L, Hq, hd])."""
    assert w.mode == "decode"
    p = oracle_projection(w, d_model, [r])
    base = int(w.cu_seqlens[r])
    n = w.row_len(r)
    tokens = base + np.arange(n, dtype=np.int64)
    k_idx = w.k_idx_f64(tokens)
    k_idx[n - 1] = gen.bf16_bits_to_f64(p["k_idx_new"][0])
    k_new = gen.bf16_bits_to_f64(w.kv_new_bits([r], "k"))[0]
    v_new = gen.bf16_bits_to_f64(w.kv_new_bits([r], "v"))[0]

    def fetch(sel):
        sel = np.asarray(sel, dtype=np.int64)
        kf, vf = w.kv_f64(base + sel)
        last = sel == n - 1
        kf[last] = k_new
        vf[last] = v_new
        return kf, vf

    res = step_row(gen.bf16_bits_to_f64(p["q_idx"][0]), k_idx, w.q_f64([r])[0], fetch, w.topk)
    # indexer entries are multiples of 1/idx_den, projected ones multiples of 1/8
    assert 8 % w.idx_den == 0
    assert_scores_exact(res["scores"], 1.0 / 64.0)
    res["idx"], res["count"] = pad_selection(res["sel"], w.topk)
    res["q_idx"], res["k_idx_new"] = p["q_idx"][0], p["k_idx_new"][0]
    return res


# ---------------------------------------------------------------------------------------------
# The distillation target and loss of eq. 4-5 on a prefill workload
# ---------------------------------------------------------------------------------------------
def oracle_distill_row(w: Workload, r: int, scale: float | None = None) -> dict:
    """fp64 eq. 4-5 for query row r of a prefill workload (row r sees tokens 0..r): A-bar_r from
    the row's per-layer queries and the shared K cache, I_r from its indexer query and K_idx, and
    KL(A-bar_r || softmax(I_r)).  scale: the attention scale of the layers' distributions (None =
    1/sqrt(head_dim); 1.0 = the unscaled form eq. 4 prints).  dict(abar, scores, kl)."""
    assert w.mode == "prefill"
    n = w.row_len(r)
    tokens = np.arange(n, dtype=np.int64)
    k = gen.bf16_bits_to_f64(w.kv_bits(tokens, "k"))
    abar = distill_target(w.q_f64([r])[0], k, scale)
    scores = index_scores(w.q_idx_f64([r])[0], w.k_idx_f64(tokens))
    return {"abar": abar, "scores": scores, "kl": distill_kl(abar, scores)}
