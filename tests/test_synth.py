"""The seeded input generator: reproducibility, rounding, ranges, distributions, needles."""
import numpy as np
import torch

import clsa_synth as cs
from clsa_synth import gen


def test_splitmix64_known_values():
    # SplitMix64 with state 0: the first outputs are published test values of the generator
    # (Steele, Lea & Flood 2014; also java.util.SplittableRandom(0).nextLong()).
    st = np.uint64(0)
    outs = []
    with np.errstate(over="ignore"):
        for i in range(3):
            outs.append(int(gen.mix(st + np.uint64(i) * gen.GAMMA)))
    assert outs[0] == 0xE220A8397B1DCDAF
    assert outs[1] == 0x6E789E6AA1B965F4
    assert outs[2] == 0x06C45D188009454F


def test_reproducible_and_seed_dependent():
    a = gen.normal_bf16(3, gen.TID_K, np.arange(1000))
    b = gen.normal_bf16(3, gen.TID_K, np.arange(1000))
    c = gen.normal_bf16(4, gen.TID_K, np.arange(1000))
    d = gen.normal_bf16(3, gen.TID_V, np.arange(1000))
    assert np.array_equal(a, b) and not np.array_equal(a, c) and not np.array_equal(a, d)
    # element values do not depend on which subset is requested
    assert np.array_equal(gen.normal_bf16(3, gen.TID_K, np.array([999, 5])), a[[999, 5]])


def test_bf16_rounding_matches_torch_round_to_nearest_even():
    rng = np.random.default_rng(0)
    x = np.concatenate([rng.standard_normal(100000).astype(np.float32),
                        (rng.standard_normal(1000) * 1e-30).astype(np.float32),
                        np.array([1.00390625, 1.01171875, -2.00390625, 0.0, -0.0], dtype=np.float32)])
    want = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(gen.f32_to_bf16_bits(x), want)


def test_uniform_int_range_and_exactness():
    v = gen.bf16_bits_to_f64(gen.uniform_int_bf16(1, gen.TID_K_IDX, np.arange(200000), -8, 8, 8))
    assert set(np.unique(v * 8).tolist()) == set(range(-8, 9))
    counts = np.bincount((v * 8 + 8).astype(int), minlength=17)
    assert counts.min() > 0.9 * 200000 / 17 and counts.max() < 1.1 * 200000 / 17
    t = gen.bf16_bits_to_f64(gen.uniform_int_bf16(1, gen.TID_K_IDX, np.arange(30000), -1, 1, 4))
    assert set(np.unique(t).tolist()) == {-0.25, 0.0, 0.25}


def test_normal_moments():
    z = gen.bf16_bits_to_f64(gen.normal_bf16(7, gen.TID_Q, np.arange(400000)))
    assert abs(z.mean()) < 0.01 and abs(z.var() - 1.0) < 0.01 and np.abs(z).max() <= 6.0


def test_needles_distinct_and_in_range():
    for n, c in [(4096, 8), (100, 100), (131072, 32)]:
        p = gen.needle_positions(5, 3, n, c)
        assert len(set(p)) == c and min(p) >= 0 and max(p) < n


def test_needle_rows_are_twice_the_query():
    w = cs.config(2)
    for r in [0, 7]:
        pos = w.needle_positions_of_row(r)
        assert len(pos) == 16
        k = w.k_idx_f64(w.cu_seqlens[r] + np.array(pos))
        assert np.array_equal(k, np.broadcast_to(2.0 * w.q_idx_f64([r])[0], k.shape))


def test_planted_needles_fill_their_range_and_join_the_drawn_ones():
    w = cs.custom(seq_lens=(3000, 2000), d_idx=64, topk=32, needles=4, seed=7, planted=((1, 100, 50),))
    pos1 = w.needle_positions_of_row(1)
    assert set(range(100, 150)) <= set(pos1) and len(pos1) == len(set(pos1)) >= 50
    assert len(w.needle_positions_of_row(0)) == 4
    k = w.k_idx_f64(w.cu_seqlens[1] + np.arange(100, 150))
    assert np.array_equal(k, np.broadcast_to(2.0 * w.q_idx_f64([1])[0], k.shape))
    # a token next to the range keeps its drawn values
    plain = cs.custom(seq_lens=(3000, 2000), d_idx=64, topk=32, needles=4, seed=7)
    t = [w.cu_seqlens[1] + 150, w.cu_seqlens[1] + 99]
    assert np.array_equal(w.k_idx_bits(t), plain.k_idx_bits(t))


def test_ragged_lengths_log_uniform():
    w = cs.config(5)
    lens = np.array(w.seq_lens)
    assert lens.min() >= 4096 and lens.max() <= 131072 and len(lens) == 64
    u = np.log(lens / 4096.0) / np.log(32.0)
    assert 0.3 < u.mean() < 0.7
    assert cs.config(5).seq_lens == w.seq_lens


def test_config_shapes():
    w3 = cs.config(3)
    assert (w3.batch, w3.max_row_len, w3.topk, w3.n_layers, w3.hq, w3.hkv, w3.d_idx) == (16, 131072, 2048, 16, 32, 8, 128)
    w4 = cs.config(4)
    assert w4.mode == "prefill" and w4.n_rows == 8192 and w4.row_len(0) == 1 and w4.row_len(8191) == 8192
