"""Pins of the fp64 oracle against facts that do not come from the oracle itself.

Routing (picx.dev summary, Architecture Overview, eq. 2) and attention (eq. 3 with the
softmax(QK^T/sqrt(d))V of the zhichai.net explainer's Background section) are checked
against closed forms, brute force on tiny inputs, hand-worked values and special cases
that reduce to a library attention routine (torch's scaled_dot_product_attention in
float64 on the CPU).  Each test is chosen so that a plausible slip in the oracle - a
dropped term, a wrong sign, a transposed operand, a wrong head map or scale - fails it.
"""
import json
import math
import os

import numpy as np
import pytest
import torch

import clsa_synth as cs
from oracle import clsa_oracle as numpy_oracle
from oracle import cpp as cpp_oracle
from oracle.workload_oracle import oracle_row

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


@pytest.fixture(params=["numpy", "cpp"])
def O(request):
    """Every primitive pin runs against both oracles (numpy, and the independent C++ one)."""
    return numpy_oracle if request.param == "numpy" else cpp_oracle


# ----------------------------------------------------------------------------- scores (a1)
def test_scores_one_hot_query_reads_one_key_column(O):
    rng = np.random.default_rng(0)
    k = rng.integers(-8, 9, size=(37, 16)) / 8.0
    for c in range(16):
        q = np.zeros(16)
        q[c] = 1.0
        assert np.array_equal(O.index_scores(q, k), k[:, c])


def test_scores_hand_worked_example(O):
    g = json.load(open(os.path.join(GOLDEN, "tiny_routing.json")))
    s = O.index_scores(np.array(g["q_idx"]), np.array(g["k_idx"]))
    assert s.tolist() == g["scores"]


def test_scores_needle_closed_form(O):
    w = cs.config(1)
    q = w.q_idx_f64([0])[0]
    needles = w.needle_positions_of_row(0)
    assert len(needles) == 8
    s = O.index_scores(q, w.k_idx_f64(needles))
    assert np.all(s == 2.0 * float(np.dot(q, q)))   # K_idx row = 2 q  ->  score = 2 |q|^2


def test_scores_sign_and_linearity(O):
    rng = np.random.default_rng(1)
    k = rng.integers(-8, 9, size=(50, 8)) / 8.0
    q = rng.integers(-8, 9, size=8) / 8.0
    assert np.array_equal(O.index_scores(-q, k), -O.index_scores(q, k))
    assert np.array_equal(O.index_scores(2 * q, k), 2 * O.index_scores(q, k))


@pytest.mark.parametrize("cfg,rows", [(1, [0]), (2, [3]), (5, [0, 7])])
def test_config_scores_exact_in_fp32(O, cfg, rows):
    """Exactness precondition of the bitwise score comparison holds on the config inputs."""
    w = cs.config(cfg)
    cu = w.cu_seqlens
    for r in rows:
        n = w.row_len(r)
        s = O.index_scores(w.q_idx_f64([r])[0], w.k_idx_f64(cu[r] + np.arange(n)))
        O.assert_scores_exact(s, 1.0 / w.idx_den ** 2)
        assert np.array_equal(s.astype(np.float32).astype(np.float64), s)


# ----------------------------------------------------------------------------- top-k (a2)
def _brute_force_selection(scores, k):
    """Token j is selected iff fewer than k tokens precede it in (score desc, index asc)."""
    n = len(scores)
    sel = []
    for j in range(n):
        rank = sum(1 for i in range(n) if scores[i] > scores[j] or (scores[i] == scores[j] and i < j))
        if rank < k:
            sel.append(j)
    return sel


def test_topk_equals_brute_force_on_tiny_inputs(O):
    rng = np.random.default_rng(2)
    for trial in range(40):
        n = int(rng.integers(1, 65))
        levels = int(rng.integers(1, 6))
        scores = rng.integers(-levels, levels + 1, size=n).astype(np.float64) * 0.5
        for k in range(1, n + 3):
            got = O.topk_select(scores, k).tolist()
            assert got == _brute_force_selection(scores.tolist(), k), (trial, n, k)


def test_topk_hand_worked_example(O):
    g = json.load(open(os.path.join(GOLDEN, "tiny_routing.json")))
    for k, want in g["selected"].items():
        assert O.topk_select(np.array(g["scores"]), int(k)).tolist() == want


def test_topk_all_equal_takes_lowest_indices(O):
    for n, k in [(10, 3), (5, 5), (4, 9)]:
        assert O.topk_select(np.zeros(n), k).tolist() == list(range(min(n, k)))


def test_topk_negative_zero_ties_with_zero(O):
    s = np.array([0.0, -0.0, -0.0, 0.0, 1.0])
    assert O.topk_select(s, 3).tolist() == [0, 1, 4]
    assert O.topk_select(-s[::-1].copy(), 2).tolist() == [1, 2]   # [-1, -0, 0, 0, -0] -> first two zeros


def test_topk_count_order_and_padding(O):
    rng = np.random.default_rng(3)
    s = rng.standard_normal(100)
    sel = O.topk_select(s, 10)
    assert len(sel) == 10 and np.all(np.diff(sel) > 0)
    assert np.min(s[sel]) >= np.max(np.delete(s, sel))
    idx, cnt = O.pad_selection(O.topk_select(s[:7], 10), 10)
    assert cnt == 7 and idx.tolist() == list(range(7)) + [-1, -1, -1]


def test_topk_permutation_invariant_on_tie_free_inputs(O):
    rng = np.random.default_rng(4)
    n, k = 500, 37
    s = rng.permutation(n).astype(np.float64) - 250.0     # distinct values
    perm = rng.permutation(n)
    base = set(O.topk_select(s, k).tolist())
    moved = set(O.topk_select(s[perm], k).tolist())
    assert {int(perm[j]) for j in moved} == base


def test_topk_permutation_on_tie_heavy_workload_scores(O):
    """Ties at the threshold are certain on the workload inputs, so lower-index-first is not
    permutation invariant; what must hold is that the tokens strictly above the k-th score map
    through the permutation and that the multiset of selected scores is unchanged."""
    w = cs.config(5)
    n = w.row_len(0)
    s = O.index_scores(w.q_idx_f64([0])[0], w.k_idx_f64(np.arange(n)))
    k = w.topk
    sel = O.topk_select(s, k)
    T = np.min(s[sel])
    assert np.sum(s == T) > np.sum(s[sel] == T)            # the threshold value is really tied
    perm = np.random.default_rng(6).permutation(n)          # new position i holds old token perm[i]
    sel_p = O.topk_select(s[perm], k)
    assert set(perm[sel_p][s[perm][sel_p] > T].tolist()) == set(sel[s[sel] > T].tolist())
    assert np.array_equal(np.sort(s[perm][sel_p]), np.sort(s[sel]))


def test_topk_two_level_ties(O):
    # ties above the threshold and at it: the three 5s are all taken, then the two lowest-index 2s
    s = np.array([2.0, 5.0, 2.0, 1.0, 5.0, 2.0, 5.0, 2.0, 0.0])
    assert O.topk_select(s, 5).tolist() == [0, 1, 2, 4, 6]
    assert O.topk_select(s, 3).tolist() == [1, 4, 6]
    assert O.topk_select(s, 8).tolist() == [0, 1, 2, 3, 4, 5, 6, 7]


def test_topk_selects_planted_needles():
    w = cs.config(1)
    res = oracle_row(w, 0)
    assert set(w.needle_positions_of_row(0)) <= set(res["sel"].tolist())
    assert res["count"] == 256


# ----------------------------------------------------------------------------- attention (a4)
def _sdpa_gqa(q, k, v, scale=None):
    """torch's float64 CPU attention with each query head reading KV head h // (Hq // Hkv)."""
    lc, hq, hd = q.shape
    m, hkv, _ = k.shape
    kk = torch.from_numpy(np.repeat(k, hq // hkv, axis=1)).permute(1, 0, 2)     # (Hq, m, hd)
    vv = torch.from_numpy(np.repeat(v, hq // hkv, axis=1)).permute(1, 0, 2)
    qq = torch.from_numpy(q).permute(1, 0, 2)                                   # (Hq, Lc, hd)
    o = torch.nn.functional.scaled_dot_product_attention(qq, kk, vv, scale=scale)
    return o.permute(1, 0, 2).numpy()


def test_attention_matches_library_routine(O):
    rng = np.random.default_rng(5)
    for lc, hq, hkv, m, hd in [(3, 8, 2, 40, 128), (1, 4, 4, 1, 16), (2, 6, 3, 129, 32)]:
        q = rng.standard_normal((lc, hq, hd))
        k = rng.standard_normal((m, hkv, hd))
        v = rng.standard_normal((m, hkv, hd))
        np.testing.assert_allclose(O.sparse_attention(q, k, v), _sdpa_gqa(q, k, v), rtol=1e-12, atol=1e-12)


def test_attention_zero_query_gives_mean_of_selected_values(O):
    rng = np.random.default_rng(6)
    k = rng.standard_normal((9, 2, 128))
    v = rng.standard_normal((9, 2, 128))
    out = O.sparse_attention(np.zeros((2, 4, 128)), k, v)
    for h in range(4):
        np.testing.assert_allclose(out[:, h, :], np.broadcast_to(v[:, h // 2, :].mean(0), (2, 128)), atol=1e-14)


def test_attention_constant_values_and_single_row(O):
    rng = np.random.default_rng(7)
    q = rng.standard_normal((2, 4, 128))
    k = rng.standard_normal((11, 1, 128))
    v = np.full((11, 1, 128), 0.375)
    np.testing.assert_allclose(O.sparse_attention(q, k, v), 0.375, atol=1e-14)
    v1 = rng.standard_normal((1, 1, 128))
    np.testing.assert_allclose(O.sparse_attention(q, k[:1], v1), np.broadcast_to(v1[0, 0], (2, 4, 128)), atol=1e-14)


def test_attention_two_rows_closed_form_pins_scale(O):
    """Two selected rows: O = sigmoid(d) V0 + (1 - sigmoid(d)) V1 with d = (q.K0 - q.K1)/sqrt(128)."""
    rng = np.random.default_rng(8)
    q = rng.standard_normal((1, 1, 128))
    k = rng.standard_normal((2, 1, 128))
    v = rng.standard_normal((2, 1, 128))
    d = float(q[0, 0] @ (k[0, 0] - k[1, 0])) / math.sqrt(128.0)
    a = 1.0 / (1.0 + math.exp(-d))
    np.testing.assert_allclose(O.sparse_attention(q, k, v)[0, 0], a * v[0, 0] + (1 - a) * v[1, 0], atol=1e-13)


def test_attention_gqa_head_map_is_contiguous_groups(O):
    rng = np.random.default_rng(9)
    hq, hkv = 32, 8
    k = rng.standard_normal((5, hkv, 128))
    v = np.zeros((5, hkv, 128))
    for g in range(hkv):
        v[:, g, :] = g
    out = O.sparse_attention(rng.standard_normal((3, hq, 128)), k, v)
    for h in range(hq):
        np.testing.assert_allclose(out[:, h, :], math.floor(h * hkv / hq), atol=1e-12)


def test_attention_dominant_logit_returns_that_row(O):
    rng = np.random.default_rng(10)
    k = rng.standard_normal((6, 1, 128))
    q = np.zeros((1, 1, 128))
    q[0, 0] = 1.0
    k[3, 0, 0] = 4000.0           # logit 4000/sqrt(128) ~ 354 above the rest
    v = rng.standard_normal((6, 1, 128))
    np.testing.assert_allclose(O.sparse_attention(q, k, v)[0, 0], v[3, 0], atol=1e-12)


def test_attention_is_a_function_of_the_selected_set(O):
    rng = np.random.default_rng(11)
    q = rng.standard_normal((2, 4, 128))
    k = rng.standard_normal((17, 2, 128))
    v = rng.standard_normal((17, 2, 128))
    p = rng.permutation(17)
    np.testing.assert_allclose(O.sparse_attention(q, k[p], v[p]), O.sparse_attention(q, k, v), atol=1e-13)


# ----------------------------------------------------------------------------- whole row (a1-a5)
def test_step_with_k_at_least_n_is_dense_attention_over_the_cache():
    w = cs.custom(seq_lens=(96,), topk=200, n_layers=3, hq=8, hkv=2, seed=12)
    res = oracle_row(w, 0)
    assert res["sel"].tolist() == list(range(96))
    kf, vf = w.kv_f64(np.arange(96))
    np.testing.assert_allclose(res["out"], _sdpa_gqa(w.q_f64([0])[0], kf, vf), rtol=1e-12, atol=1e-12)


def test_step_every_layer_uses_the_same_selection():
    w = cs.custom(seq_lens=(300,), topk=20, n_layers=4, hq=4, hkv=2, seed=13)
    res = oracle_row(w, 0)
    kf, vf = w.kv_f64(res["sel"])
    q = w.q_f64([0])[0]
    for layer in range(4):
        np.testing.assert_allclose(res["out"][layer], _sdpa_gqa(q[layer:layer + 1], kf, vf)[0], atol=1e-12)


def test_prefill_row_equals_decode_of_the_truncated_sequence(O):
    wp = cs.custom(mode="prefill", seq_lens=(64,), topk=16, n_layers=2, hq=4, hkv=1, seed=14)
    for t in [0, 5, 15, 16, 40, 63]:
        res = oracle_row(wp, t)
        assert res["count"] == min(16, t + 1)
        s = O.index_scores(wp.q_idx_f64([t])[0], wp.k_idx_f64(np.arange(t + 1)))
        assert res["sel"].tolist() == _brute_force_selection(s.tolist(), 16)


def test_prefill_needles_against_last_row(O):
    w = cs.config(4)
    pos = w.needle_positions_of_row(w.n_rows - 1)
    assert len(pos) == 16
    q = w.q_idx_f64([w.n_rows - 1])[0]
    s = O.index_scores(q, w.k_idx_f64(np.arange(8192)))
    sel = set(O.topk_select(s, 2048).tolist())
    assert set(pos) <= sel
