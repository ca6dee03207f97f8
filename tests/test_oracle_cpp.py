"""The C++ fp64 oracle against the Python one, and its generator against the Python generator.

The two oracles are written independently (the C++ one regenerates its inputs from the generator
definition itself), so bitwise-equal selections and fp64-equal outputs on every workload pin each
against a slip in the other: a wrong needle, head map, scale, tie rule or sum order shows here.
"""
import numpy as np
import pytest

import clsa_synth as cs
from clsa_synth import gen
from oracle import cpp as C
from oracle.workload_oracle import oracle_row as numpy_oracle_row

pytestmark = pytest.mark.filterwarnings("ignore::RuntimeWarning")


def test_generator_uniform_and_normal_match_python_bitwise():
    rng = np.random.default_rng(5)
    for seed in (0, 1, 3, 5, 2**63 + 17):
        idx = rng.integers(0, 2**40, size=200)
        for tid, lo, hi, den in ((gen.TID_Q_IDX, -8, 8, 8), (gen.TID_K_IDX, -1, 1, 4)):
            want = gen.uniform_int_bf16(seed, tid, idx, lo, hi, den)
            got = [C.gen_uniform(seed, tid, int(i), lo, hi, den) for i in idx]
            assert np.array_equal(np.asarray(got, dtype=np.uint16), want)
        for tid in (gen.TID_Q, gen.TID_K, gen.TID_V):
            want = gen.normal_bf16(seed, tid, idx)
            got = [C.gen_normal(seed, tid, int(i)) for i in idx]
            assert np.array_equal(np.asarray(got, dtype=np.uint16), want)


def test_generator_needles_match_python():
    for seed, row, n, count in ((1, 0, 4096, 8), (3, 15, 131072, 32), (4, 0, 8192, 16), (9, 2, 40, 40)):
        assert C.gen_needles(seed, row, n, count) == gen.needle_positions(seed, row, n, count)


ROWS = [(1, [0]), (2, [3]), (3, [5]), (4, [0, 1, 2046, 2047, 2048, 5000, 8191]), (5, [0, 1, 63])]


@pytest.mark.parametrize("cfg,rows", ROWS)
def test_cpp_oracle_equals_numpy_oracle_on_workload_rows(cfg, rows):
    w = cs.config(cfg)
    for r in rows:
        a = C.oracle_row(w, r, with_scores=True)
        b = numpy_oracle_row(w, r)
        assert np.array_equal(a["scores"], b["scores"]), (cfg, r)          # exact inputs, exact sums
        assert a["count"] == b["count"] and np.array_equal(a["idx"], b["idx"]), (cfg, r)
        np.testing.assert_allclose(a["out"], b["out"], rtol=0, atol=1e-12, err_msg=f"cfg {cfg} row {r}")


def test_threaded_driver_equals_single_rows():
    w = cs.config(2)
    rows = [0, 7, 3, 5]
    res, secs = C.oracle_rows_timed(w, rows, threads=3)
    assert secs > 0
    for i, r in enumerate(rows):
        one = C.oracle_row(w, r)
        assert np.array_equal(res["idx"][i], one["idx"]) and res["count"][i] == one["count"]
        assert np.array_equal(res["out"][i], one["out"])


def test_needles_selected_by_cpp_oracle():
    w = cs.config(1)
    sel = set(C.oracle_row(w, 0)["idx"].tolist())
    assert set(w.needle_positions_of_row(0)) <= sel


def test_cpp_oracle_rejects_more_needles_than_tokens():
    w = cs.custom(seq_lens=(1, 50), needles=4, seed=1)
    with pytest.raises(AssertionError):
        C.oracle_row(w, 0)
    with pytest.raises(ValueError):
        C.gen_needles(1, 0, 1, 4)
