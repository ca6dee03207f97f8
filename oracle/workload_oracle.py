"""Oracle results for rows of a synthetic workload (test infrastructure only).

Regenerates, on the host, exactly the inputs a query row needs - its indexer query,
the indexer keys of the tokens it sees, its per-layer queries and only the selected
K/V rows - and runs the fp64 oracle on them.  Inputs come from ``clsa_synth`` alone.
"""
from __future__ import annotations

import numpy as np

from clsa_synth import Workload

from .clsa_oracle import assert_scores_exact, pad_selection, step_row


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
