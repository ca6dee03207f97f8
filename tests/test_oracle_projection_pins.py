"""Pins of the oracle of the step before the routing: the indexer projections of the new token
(picx.dev summary, Methodology > Architecture Overview, eq. 1: Q_idx = H W_idx^Q,
K_idx = H W_idx^K), the rounding of their results to bf16, and the decode step that appends the
new token to the caches before scoring.  Each pin comes from outside the oracle: one-hot inputs,
exact rational arithmetic on tiny inputs, hand-worked rounding cases, an independent rounding
formula, and closed forms of the appended step.
"""
from fractions import Fraction

import numpy as np
import pytest

import clsa_synth as cs
from clsa_synth import gen
from oracle import clsa_oracle as O
from oracle.workload_oracle import oracle_projection, oracle_row, oracle_row_projected


# ----------------------------------------------------------------------------- eq. 1
def test_projection_one_hot_hidden_state_reads_one_weight_column():
    rng = np.random.default_rng(0)
    w = rng.integers(-8, 9, size=(16, 40)) / 8.0          # [d_idx, d_model]
    for c in range(40):
        h = np.zeros((1, 40))
        h[0, c] = 1.0
        assert np.array_equal(O.index_projection(h, w)[0], w[:, c])


def test_projection_equals_exact_rational_sums():
    rng = np.random.default_rng(1)
    h = rng.integers(-3, 4, size=(3, 24))
    w = rng.integers(-8, 9, size=(5, 24))
    got = O.index_projection(h.astype(np.float64), w / 8.0)
    for t in range(3):
        for j in range(5):
            exact = sum(Fraction(int(h[t, c])) * Fraction(int(w[j, c]), 8) for c in range(24))
            assert Fraction(got[t, j]) == exact


def test_projection_rows_are_independent():
    rng = np.random.default_rng(2)
    h = rng.integers(-1, 2, size=(6, 32)).astype(np.float64)
    w = rng.integers(-1, 2, size=(8, 32)) / 8.0
    full = O.index_projection(h, w)
    for t in range(6):
        assert np.array_equal(O.index_projection(h[t:t + 1], w)[0], full[t])


# ----------------------------------------------------------------------------- bf16 rounding
def test_round_bf16_matches_fp32_bit_rounding_on_fp32_values():
    rng = np.random.default_rng(3)
    x = (rng.standard_normal(200000) * np.exp2(rng.integers(-20, 20, 200000))).astype(np.float32)
    assert np.array_equal(O.round_bf16_bits(x.astype(np.float64)), gen.f32_to_bf16_bits(x))


@pytest.mark.parametrize("x,bits", [
    (1.0, 0x3F80),
    (1.0 + 2.0 ** -8, 0x3F80),                 # halfway between 1 and 1 + 2^-7: to even
    (1.0 + 3 * 2.0 ** -8, 0x3F82),             # halfway between 1 + 2^-7 and 1 + 2^-6: to even
    (-(1.0 + 2.0 ** -8), 0xBF80),
    (1.0 + 2.0 ** -8 + 2.0 ** -40, 0x3F81),    # just above halfway; lost if rounded via fp32 first
    (255.5, 0x4380),                           # 255.5 needs 9 bits: halfway, to even 256
    (254.5, 0x437E),                           # halfway between 254 and 255: to even 254
    (-3.0, 0xC040),
    (0.0, 0x0000),
])
def test_round_bf16_hand_worked_cases(x, bits):
    assert int(O.round_bf16_bits(np.array([x]))[0]) == bits


# ----------------------------------------------------------------------------- appended step
def _tiny(seed=5, topk=3, n=(9, 6)):
    return cs.custom(seq_lens=n, d_idx=64, topk=topk, n_layers=2, hq=4, hkv=2, seed=seed)


def test_projected_scores_equal_exact_rational_scores():
    w = _tiny()
    d_model = 32
    for r in range(w.batch):
        res = oracle_row_projected(w, r, d_model)
        n = w.row_len(r)
        base = int(w.cu_seqlens[r])
        h = [Fraction(int(v)) for v in gen.bf16_bits_to_f64(w.h_new_bits([r], d_model))[0]]
        wq = gen.bf16_bits_to_f64(w.w_idx_bits("q", d_model))
        wk = gen.bf16_bits_to_f64(w.w_idx_bits("k", d_model))
        q = [sum(h[c] * Fraction(wq[j, c]) for c in range(d_model)) for j in range(64)]
        knew = [sum(h[c] * Fraction(wk[j, c]) for c in range(d_model)) for j in range(64)]
        # the sums are small multiples of 1/8: exactly representable in bf16, so rounding is a no-op
        assert all(abs(v) < 32 for v in q + knew)
        kidx = w.k_idx_f64(base + np.arange(n))
        for j in range(n):
            key = knew if j == n - 1 else [Fraction(v) for v in kidx[j]]
            assert Fraction(res["scores"][j]) == sum(a * b for a, b in zip(q, key))


def test_projected_step_with_top1_new_token_returns_its_value_row():
    """With k = 1 the selected set is the single best token; when that is the appended token,
    every (layer, head) output is exactly its V row (a softmax over one element)."""
    hits = 0
    for seed in range(1, 40):
        w = _tiny(seed=seed, topk=1, n=(50,))
        res = oracle_row_projected(w, 0, 1024)
        if res["sel"].tolist() != [49]:
            continue
        hits += 1
        v_new = gen.bf16_bits_to_f64(w.kv_new_bits([0], "v"))[0]
        for h in range(w.hq):
            g = h // (w.hq // w.hkv)
            assert np.array_equal(res["out"][:, h, :], np.broadcast_to(v_new[g], res["out"][:, h, :].shape))
    assert hits >= 3


def test_projected_step_with_k_at_least_n_attends_to_every_token_including_the_new_one():
    w = _tiny(topk=64, n=(20,))
    res = oracle_row_projected(w, 0, 32)
    assert res["sel"].tolist() == list(range(20))
    q = w.q_f64([0])[0]
    k, v = w.kv_f64(np.arange(20))
    k[19] = gen.bf16_bits_to_f64(w.kv_new_bits([0], "k"))[0]
    v[19] = gen.bf16_bits_to_f64(w.kv_new_bits([0], "v"))[0]
    assert np.allclose(res["out"], O.sparse_attention(q, k, v), rtol=0, atol=1e-13)
    # and differs from the step over the cache without the append
    assert not np.allclose(res["out"], oracle_row(w, 0)["out"], rtol=0, atol=1e-6)


def test_projection_of_the_workload_is_exact_in_fp32():
    """Precondition of bit-exact parity: every partial sum is a multiple of 1/8 below 2^21."""
    w = cs.config(3)
    d_model = 4096
    h = gen.bf16_bits_to_f64(w.h_new_bits(np.arange(w.batch), d_model))
    assert set(np.unique(h)) <= {-1.0, 0.0, 1.0}
    wq = gen.bf16_bits_to_f64(w.w_idx_bits("q", d_model))
    assert set(np.unique(wq * 8)) <= {-1.0, 0.0, 1.0}
    p = oracle_projection(w, d_model)
    q = gen.bf16_bits_to_f64(p["q_idx"])
    assert np.all(q * 8 == np.round(q * 8)) and np.abs(q).max() <= d_model / 8
