"""Pins of the oracle of the per-layer routing ablation (zhichai.net explainer, Ablations: the
variant without the cross-layer shared index recomputes the routing in every layer; picx.dev
summary, Complexity Comparison: a per-layer indexer costs eta L N instead of eta N).

``oracle_row_layer_routing`` scores every layer with its OWN indexer query, selects that layer's
own set and attends with that layer's query over it.  The pins below fail on the plausible slips:
scoring every layer with the shared ``q_idx`` (the one-hot test), attending layer l over layer 0's
selection or with the wrong layer's query (the brute-force attention test), and mixing the layers
up (the reduction to the shared-routing oracle, and the one-layer change test).  The C++ oracle's
own implementation of the ablation is checked against the numpy one on workload rows.
"""
import math

import numpy as np
import pytest

import clsa_synth as cs
from oracle import cpp as C
from oracle.workload_oracle import oracle_row, oracle_row_layer_routing


class _Arrays:
    """A duck-typed decode workload of one sequence holding explicit fp64 arrays, with the
    methods the oracle reads."""

    def __init__(self, k_idx, q_idx_layers, q, k, v, topk, q_idx=None):
        self.k_idx = np.asarray(k_idx, dtype=np.float64)          # [n, d_idx]
        self.q_idx_layers = np.asarray(q_idx_layers, dtype=np.float64)  # [L, d_idx]
        self.q = np.asarray(q, dtype=np.float64)                  # [L, Hq, hd]
        self.k = np.asarray(k, dtype=np.float64)                  # [n, Hkv, hd]
        self.v = np.asarray(v, dtype=np.float64)
        self.topk = topk
        self.n_layers = self.q.shape[0]
        self.cu_seqlens = np.array([0, self.k_idx.shape[0]], dtype=np.int32)

    def row_seq(self, r):
        return 0

    def row_len(self, r):
        return self.k_idx.shape[0]

    def k_idx_f64(self, tokens):
        return self.k_idx[np.asarray(tokens)]

    def q_idx_layer_f64(self, rows, layer):
        return self.q_idx_layers[layer][None, :]

    def q_f64(self, rows):
        return self.q[None]

    def kv_f64(self, tokens):
        t = np.asarray(tokens)
        return self.k[t], self.v[t]


def _brute_attention(qv, k_rows, v_rows, scale):
    """softmax(q . k * scale) v with Python floats, one (layer, head) at a time."""
    logits = [scale * sum(a * b for a, b in zip(qv, kr)) for kr in k_rows]
    mx = max(logits)
    p = [math.exp(x - mx) for x in logits]
    den = sum(p)
    return np.array([sum(pi * vr[d] for pi, vr in zip(p, v_rows)) / den for d in range(len(qv))])


def _tiny(seed, n=40, d=8, L=3, hq=4, hkv=2, hd=8, topk=5):
    """Indexer keys whose columns each hold a permutation of distinct eighths (no ties in any
    one-hot score), one-hot per-layer indexer queries on distinct columns, normal Q/K/V."""
    rng = np.random.default_rng(seed)
    k_idx = np.stack([rng.permutation(n) for _ in range(d)], axis=1).astype(np.float64) / 8.0
    cols = rng.choice(d, L, replace=False)
    q_idx = np.zeros((L, d))
    q_idx[np.arange(L), cols] = 1.0
    q = rng.standard_normal((L, hq, hd))
    k = rng.standard_normal((n, hkv, hd))
    v = rng.standard_normal((n, hkv, hd))
    return _Arrays(k_idx, q_idx, q, k, v, topk), cols


def test_one_hot_layer_queries_select_their_own_column():
    """Layer l's query is one-hot on column c_l, so its selection is the top-k of that column of
    K_idx alone (Python's sort, ascending ids).  Scoring every layer with one shared query would
    give every layer the same set."""
    w, cols = _tiny(3)
    res = oracle_row_layer_routing(w, 0)
    sets = []
    for l, c in enumerate(cols):
        col = w.k_idx[:, c].tolist()
        want = sorted(sorted(range(len(col)), key=lambda j: (-col[j], j))[: w.topk])
        assert res["count"][l] == w.topk
        assert res["idx"][l].tolist() == want, f"layer {l}"
        sets.append(tuple(want))
    assert len(set(sets)) == len(sets), "the layers' selections must differ in this case"


def test_layer_output_is_attention_over_its_own_selection_with_its_own_query():
    """out[l] is softmax(q[l] K_{S_l}^T / sqrt(hd)) V_{S_l} for each head (contiguous GQA groups),
    by brute force; attending layer l over layer 0's set, or with layer 0's query, differs."""
    w, cols = _tiny(4)
    res = oracle_row_layer_routing(w, 0)
    L, hq, hd = w.q.shape
    hkv = w.k.shape[1]
    scale = 1.0 / math.sqrt(hd)
    for l in range(L):
        sel = res["idx"][l][: res["count"][l]]
        for h in range(hq):
            g = h // (hq // hkv)
            want = _brute_attention(w.q[l, h], w.k[sel, g], w.v[sel, g], scale)
            assert np.allclose(res["out"][l, h], want, rtol=0, atol=1e-12), (l, h)
    sel0 = res["idx"][0][: res["count"][0]]
    for l in range(1, L):
        wrong_set = _brute_attention(w.q[l, 0], w.k[sel0, 0], w.v[sel0, 0], scale)
        sel = res["idx"][l][: res["count"][l]]
        wrong_query = _brute_attention(w.q[0, 0], w.k[sel, 0], w.v[sel, 0], scale)
        assert not np.allclose(res["out"][l, 0], wrong_set, rtol=0, atol=1e-6)
        assert not np.allclose(res["out"][l, 0], wrong_query, rtol=0, atol=1e-6)


def test_changing_one_layer_query_changes_only_that_layer():
    w, cols = _tiny(5)
    a = oracle_row_layer_routing(w, 0)
    q_idx2 = w.q_idx_layers.copy()
    free = [c for c in range(w.k_idx.shape[1]) if c not in cols]
    q_idx2[1] = 0.0
    q_idx2[1, free[0]] = 1.0
    w2 = _Arrays(w.k_idx, q_idx2, w.q, w.k, w.v, w.topk)
    b = oracle_row_layer_routing(w2, 0)
    for l in (0, 2):
        assert np.array_equal(a["idx"][l], b["idx"][l]) and np.array_equal(a["out"][l], b["out"][l])
    assert not np.array_equal(a["idx"][1], b["idx"][1])
    assert not np.allclose(a["out"][1], b["out"][1], rtol=0, atol=1e-9)


class _SharedQuery:
    """A workload whose per-layer indexer queries are all its shared q_idx."""

    def __init__(self, w):
        self._w = w

    def __getattr__(self, name):
        return getattr(self._w, name)

    def q_idx_layer_f64(self, rows, layer):
        return self._w.q_idx_f64(rows)


_TIES = cs.custom(seq_lens=(3000, 9000), d_idx=128, topk=256, n_layers=4, hq=16, hkv=4, idx_lo=-1, idx_hi=1,
                  idx_den=4, needles=0, seed=19, name="routing_ties")
_EIGHTHS = cs.custom(seq_lens=(5000, 2000), d_idx=128, topk=512, n_layers=3, hq=8, hkv=2, needles=4, seed=23,
                     name="routing_eighths")


@pytest.mark.parametrize("w,r", [(cs.config(1), 0), (_EIGHTHS, 1)], ids=["decode_b1_n4k", "eighths"])
def test_identical_layer_queries_reduce_to_shared_routing(w, r):
    """With every layer's indexer query equal to the shared one, each layer selects the shared
    set and its output is the shared-routing oracle's output of that layer."""
    res = oracle_row_layer_routing(_SharedQuery(w), r)
    ref = oracle_row(w, r)
    for l in range(w.n_layers):
        assert res["count"][l] == ref["count"]
        assert np.array_equal(res["idx"][l], ref["idx"]), l
        np.testing.assert_allclose(res["out"][l], ref["out"][l], rtol=0, atol=1e-13)


def test_workload_layers_route_differently():
    """On a workload the layers' own indexer queries give different selections."""
    w = cs.config(1)
    res = oracle_row_layer_routing(w, 0)
    assert len({tuple(x) for x in res["idx"]}) == w.n_layers


@pytest.mark.filterwarnings("ignore::RuntimeWarning")
@pytest.mark.parametrize("w,rows", [(cs.config(1), [0]), (_EIGHTHS, [0, 1]), (_TIES, [1, 0])],
                         ids=["decode_b1_n4k", "eighths", "ties"])
def test_cpp_layer_routing_equals_numpy(w, rows):
    """The C++ oracle's per-layer routing (its own generator of the per-layer indexer queries)
    against the numpy oracle, on eighths with needles and on tie-heavy {-1, 0, 1} / 4 entries:
    selections bitwise, outputs within 1e-12; the threaded driver against the single rows."""
    cfg = w.name
    many = C.oracle_rows_layer_routing(w, rows, threads=2)
    for i, r in enumerate(rows):
        a = C.oracle_row_layer_routing(w, r)
        b = oracle_row_layer_routing(w, r)
        assert np.array_equal(a["count"], b["count"]) and np.array_equal(a["idx"], b["idx"]), (cfg, r)
        np.testing.assert_allclose(a["out"], b["out"], rtol=0, atol=1e-12)
        assert np.array_equal(many["idx"][i], a["idx"]) and np.array_equal(many["out"][i], a["out"])
