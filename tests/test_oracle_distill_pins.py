"""Pins of the oracle of the multi-layer distillation target and loss (picx.dev summary,
Methodology, Multi-Layer Distillation, eq. 4-5): A-bar_t = mean over layers and heads of the
attention distributions, and KL(A-bar_t || softmax(I_t)).  Pinned against library routines
(scipy's softmax and relative entropy), closed forms, brute force on tiny inputs and invariants,
chosen so that a dropped scale, a wrong head map, a flipped KL direction or a missing average
fails one of them.
"""
import math

import numpy as np
import pytest
from scipy.special import softmax
from scipy.stats import entropy

import clsa_synth as cs
from oracle import clsa_oracle as O
from oracle.workload_oracle import oracle_distill_row


def _rand(seed, L=2, hq=4, hkv=2, n=9, hd=16):
    rng = np.random.default_rng(seed)
    return rng.standard_normal((L, hq, hd)), rng.standard_normal((n, hkv, hd))


def test_target_single_head_is_the_library_softmax_with_the_attention_scale():
    q, k = _rand(0, L=1, hq=1, hkv=1, n=13, hd=32)
    ref = softmax(k[:, 0, :] @ q[0, 0] / math.sqrt(32))
    assert np.allclose(O.distill_target(q, k), ref, rtol=0, atol=1e-15)


def test_target_two_keys_closed_form_fixes_the_scale():
    hd = 128
    q = np.zeros((1, 1, hd))
    q[0, 0, 0] = 1.0
    k = np.zeros((2, 1, hd))
    k[0, 0, 0] = math.sqrt(hd) * math.log(3.0)   # logit ln 3 after the 1/sqrt(128) scale
    assert np.allclose(O.distill_target(q, k), [0.75, 0.25], rtol=0, atol=1e-15)


def test_target_unscaled_form_of_the_page():
    """eq. 4 prints softmax(Q K^T) with no scale; the oracle's scale argument gives that form
    (scale = 1): the library softmax of the raw products, and the two-key closed form with the
    raw logit ln 3."""
    q, k = _rand(6, L=1, hq=1, hkv=1, n=13, hd=32)
    assert np.allclose(O.distill_target(q, k, scale=1.0), softmax(k[:, 0, :] @ q[0, 0]), rtol=0, atol=1e-15)
    qq = np.zeros((1, 1, 128))
    qq[0, 0, 0] = 1.0
    kk = np.zeros((2, 1, 128))
    kk[0, 0, 0] = math.log(3.0)
    assert np.allclose(O.distill_target(qq, kk, scale=1.0), [0.75, 0.25], rtol=0, atol=1e-15)
    # the default (1/sqrt(head_dim)) differs from it
    assert not np.allclose(O.distill_target(qq, kk), [0.75, 0.25], rtol=0, atol=1e-3)


def test_workload_row_with_the_unscaled_form():
    """oracle_distill_row(scale=1) is the target of the raw products q . k over the row's keys."""
    w = cs.custom(mode="prefill", seq_lens=(200,), d_idx=64, topk=32, n_layers=2, hq=4, hkv=2, seed=13)
    from clsa_synth import gen
    r = 150
    d = oracle_distill_row(w, r, scale=1.0)
    k = gen.bf16_bits_to_f64(w.kv_bits(np.arange(r + 1), "k"))
    q = w.q_f64([r])[0]
    per = [softmax(k[:, h // 2, :] @ q[l, h]) for l in range(2) for h in range(4)]
    assert np.allclose(d["abar"], np.mean(per, axis=0), rtol=0, atol=1e-15)


def test_target_is_a_distribution_and_averages_layers_and_heads():
    q, k = _rand(1, L=3, hq=6, hkv=3, n=11)
    a = O.distill_target(q, k)
    assert np.all(a > 0) and abs(a.sum() - 1.0) < 1e-14
    # the average of the per-(layer, head) distributions, each from the library softmax
    group = 2
    per = [softmax(k[:, h // group, :] @ q[l, h] / 4.0) for l in range(3) for h in range(6)]
    assert np.allclose(a, np.mean(per, axis=0), rtol=0, atol=1e-15)


def test_target_identical_heads_equal_one_head():
    q, k = _rand(2, L=1, hq=1, hkv=1, n=7)
    q4 = np.broadcast_to(q, (3, 4, q.shape[2])).copy()
    k2 = np.broadcast_to(k, (7, 2, k.shape[2])).copy()
    assert np.allclose(O.distill_target(q4, k2), O.distill_target(q, k), rtol=0, atol=1e-15)


def test_target_zero_queries_give_the_uniform_distribution():
    _, k = _rand(3, n=10)
    assert np.allclose(O.distill_target(np.zeros((2, 4, 16)), k), np.full(10, 0.1), rtol=0, atol=1e-15)


def test_target_head_map_is_contiguous_groups():
    """Only query heads 0 and 1 (group 0 under the contiguous map) look for key 5 of KV head 0;
    KV head 1 is zero.  Contiguous groups put both on KV head 0 (A-bar[5] ~ 2/4); an interleaved
    map would send head 1 to KV head 1 (A-bar[5] ~ 1/4)."""
    hd, n = 16, 8
    k = np.zeros((n, 2, hd))
    k[5, 0, 0] = 40.0
    q = np.zeros((1, 4, hd))
    q[0, 0, 0] = q[0, 1, 0] = 40.0
    a = O.distill_target(q, k)
    assert abs(a[5] - (2 / 4 + 2 / 4 / n)) < 1e-6


def test_kl_is_the_library_relative_entropy_and_has_the_right_direction():
    rng = np.random.default_rng(4)
    for n in (1, 2, 17, 300):
        a = rng.random(n) + 0.01
        a /= a.sum()
        s = rng.standard_normal(n) * 3
        assert math.isclose(O.distill_kl(a, s), entropy(a, softmax(s)), rel_tol=1e-12, abs_tol=1e-14)
    # the two directions differ: KL(P||Q) != KL(Q||P) in general
    a = np.array([0.9, 0.05, 0.05])
    s = np.log([0.2, 0.4, 0.4])
    assert not math.isclose(O.distill_kl(a, s), entropy(softmax(s), a), rel_tol=1e-3)


def test_kl_closed_forms():
    rng = np.random.default_rng(5)
    s = rng.standard_normal(12) * 2
    # uniform A-bar: KL = -log n - mean(log softmax(I))
    u = np.full(12, 1 / 12)
    assert math.isclose(O.distill_kl(u, s), -math.log(12) - np.mean(np.log(softmax(s))), rel_tol=1e-12)
    # matching distributions (scores = log A-bar + c): KL = 0
    a = softmax(rng.standard_normal(12))
    assert abs(O.distill_kl(a, np.log(a) + 7.5)) < 1e-14
    # a single visible token: KL = 0
    assert O.distill_kl(np.array([1.0]), np.array([3.0])) == 0.0


def test_kl_brute_force_with_python_floats():
    a = [0.5, 0.25, 0.125, 0.125]
    s = [1.0, -2.0, 0.5, 3.0]
    lse = math.log(sum(math.exp(x) for x in s))
    ref = sum(ai * (math.log(ai) - (si - lse)) for ai, si in zip(a, s))
    assert math.isclose(O.distill_kl(np.array(a), np.array(s)), ref, rel_tol=1e-14)


@pytest.mark.parametrize("r", [0, 1, 64, 300])
def test_workload_row_uses_only_its_visible_tokens(r):
    """Row r of the prefill workload sees tokens 0..r: its A-bar has r + 1 entries and equals the
    target computed from exactly those keys; row 0 has KL 0 (one token)."""
    w = cs.custom(mode="prefill", seq_lens=(400,), d_idx=64, topk=32, n_layers=2, hq=8, hkv=2, seed=9)
    d = oracle_distill_row(w, r)
    assert d["abar"].shape == (r + 1,) and abs(d["abar"].sum() - 1) < 1e-13
    from clsa_synth import gen
    k = gen.bf16_bits_to_f64(w.kv_bits(np.arange(r + 1), "k"))
    assert np.allclose(d["abar"], O.distill_target(w.q_f64([r])[0], k), rtol=0, atol=0)
    assert d["kl"] >= -1e-12
    if r == 0:
        assert d["kl"] == 0.0
