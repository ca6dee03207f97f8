"""Parity of clsa_index_project (the new token's indexer projections, eq. 1 of the picx.dev
summary's Architecture Overview, and its append to the caches) and of the decode step that
follows it, with the fp64 oracle.  Projections and appended rows must match bit for bit on the
workload inputs (every partial sum is exact in fp32 there); on general normal inputs the bf16
results may differ from the rounding of the exact sum by one unit in the last place.
"""
import contextlib

import numpy as np
import pytest
import torch

import clsa_synth as cs
import cross_layer_token_amd as clsa
from _gpu_helpers import assert_outputs_close, bf16_dev_to_f64, device_workload, dims_of, rows_of, workspace
from clsa_synth import gen
from clsa_synth.device import fill_normal
from oracle import clsa_oracle as O
from oracle.workload_oracle import oracle_projection, oracle_row_projected

pytestmark = pytest.mark.gpu

D_MODEL = 4096


def _say(*a):
    print(*a, flush=True)


def _u16(t: torch.Tensor) -> np.ndarray:
    return t.cpu().numpy().view(np.uint16)


@contextlib.contextmanager
def _restored_new_rows(dw):
    """The append overwrites each sequence's last row of k_idx / k_cache / v_cache in the shared
    resident workload; put the generated rows back afterwards."""
    w = dw.w
    rows = torch.tensor([w.new_token(b) for b in range(w.batch)], dtype=torch.int64, device="cuda")
    saved = [(t, t[rows].clone()) for t in (dw.k_idx, dw.k_cache, dw.v_cache)]
    try:
        yield rows
    finally:
        for t, s in saved:
            t[rows] = s
        torch.cuda.synchronize()


def _project(dw, d_model, with_kv=True, inputs=None):
    w = dw.w
    p = inputs if inputs is not None else dw.projection_inputs(d_model)
    q_idx = torch.full((w.batch, w.d_idx), -1, dtype=torch.int16, device="cuda")
    kv = (p["k_new"], p["v_new"], dw.k_cache, dw.v_cache) if with_kv else (None, None, None, None)
    clsa.index_project(dims_of(dw), rows_of(dw), d_model, p["h"], p["w_q_idx"], p["w_k_idx"], dw.cu_seqlens, q_idx,
                       dw.k_idx, *kv)
    torch.cuda.synchronize()
    return q_idx


@pytest.mark.parametrize("cfg", [1, 3])
def test_projection_inputs_device_matches_host(cfg):
    w = cs.config(cfg)
    dw = device_workload(w)
    p = dw.projection_inputs(D_MODEL)
    assert np.array_equal(_u16(p["h"]), w.h_new_bits(np.arange(w.batch), D_MODEL))
    assert np.array_equal(_u16(p["w_q_idx"]), w.w_idx_bits("q", D_MODEL))
    assert np.array_equal(_u16(p["w_k_idx"]), w.w_idx_bits("k", D_MODEL))
    assert np.array_equal(_u16(p["k_new"]), w.kv_new_bits(np.arange(w.batch), "k"))
    assert np.array_equal(_u16(p["v_new"]), w.kv_new_bits(np.arange(w.batch), "v"))


@pytest.mark.parametrize("cfg,d_model", [(1, 32), (1, 4096), (2, 4192), (2, 8224), (3, 4096), (5, 4096)])
def test_index_project_bitwise(cfg, d_model):
    """d_model 32 (one slice), 4096 (one round of loads), 4192 (a ragged last round) and 8224 (two
    rounds plus a ragged one); batches of 1, 8, 16 and 64 sequences."""
    w = cs.config(cfg)
    dw = device_workload(w)
    _say(f"index_project cfg{cfg} B={w.batch} d_idx={w.d_idx} d_model={d_model}")
    ref = oracle_projection(w, d_model)
    with _restored_new_rows(dw) as new_rows:
        before = {b: int(x) for b, x in enumerate(new_rows.tolist())}
        q_idx = _project(dw, d_model)
        assert np.array_equal(_u16(q_idx), ref["q_idx"])
        assert np.array_equal(_u16(dw.k_idx[new_rows]), ref["k_idx_new"])
        assert np.array_equal(_u16(dw.k_cache[new_rows]), w.kv_new_bits(np.arange(w.batch), "k"))
        assert np.array_equal(_u16(dw.v_cache[new_rows]), w.kv_new_bits(np.arange(w.batch), "v"))
        # neighbouring rows (the previous token of each sequence, and the first) are untouched
        others = sorted({max(int(w.cu_seqlens[b]), before[b] - 1) for b in range(w.batch)} | {0})
        others = [t for t in others if t not in before.values()]
        ot = torch.tensor(others, dtype=torch.int64, device="cuda")
        assert np.array_equal(_u16(dw.k_idx[ot]), w.k_idx_bits(others))
        assert np.array_equal(_u16(dw.k_cache[ot]), w.kv_bits(others, "k"))
        assert np.array_equal(_u16(dw.v_cache[ot]), w.kv_bits(others, "v"))


def test_index_project_without_kv_leaves_the_caches_alone():
    w = cs.config(2)
    dw = device_workload(w)
    with _restored_new_rows(dw) as new_rows:
        _project(dw, D_MODEL, with_kv=False)
        toks = new_rows.cpu().numpy()
        assert np.array_equal(_u16(dw.k_cache[new_rows]), w.kv_bits(toks, "k"))
        assert np.array_equal(_u16(dw.v_cache[new_rows]), w.kv_bits(toks, "v"))
        assert np.array_equal(_u16(dw.k_idx[new_rows]), oracle_projection(w, D_MODEL)["k_idx_new"])


def test_index_project_ragged_batch_tiles():
    """17 sequences: a second tile of sequences holding a single one."""
    w = cs.custom(seq_lens=[300 + 37 * i for i in range(17)], d_idx=128, topk=64, n_layers=2, hq=8, hkv=2, seed=23,
                  name="b17")
    dw = device_workload(w)
    ref = oracle_projection(w, 1024)
    with _restored_new_rows(dw) as new_rows:
        q_idx = _project(dw, 1024)
        assert np.array_equal(_u16(q_idx), ref["q_idx"])
        assert np.array_equal(_u16(dw.k_idx[new_rows]), ref["k_idx_new"])
        assert np.array_equal(_u16(dw.v_cache[new_rows]), w.kv_new_bits(np.arange(17), "v"))


def test_index_project_normal_inputs_within_one_ulp():
    """Inputs whose sums are not exact in fp32: the fp32 sum in fixed order, rounded once to bf16,
    is at most one bf16 unit from the rounding of the exact sum."""
    w = cs.config(3)
    dw = device_workload(w)
    p = dw.projection_inputs(D_MODEL)
    seed = 991
    for key, tid in (("h", 101), ("w_q_idx", 102), ("w_k_idx", 103)):
        fill_normal(p[key], seed, tid)
    torch.cuda.synchronize()
    h = gen.bf16_bits_to_f64(gen.normal_bf16(seed, 101, np.arange(w.batch * D_MODEL))).reshape(w.batch, D_MODEL)
    wq = gen.bf16_bits_to_f64(gen.normal_bf16(seed, 102, np.arange(w.d_idx * D_MODEL))).reshape(w.d_idx, D_MODEL)
    wk = gen.bf16_bits_to_f64(gen.normal_bf16(seed, 103, np.arange(w.d_idx * D_MODEL))).reshape(w.d_idx, D_MODEL)
    with _restored_new_rows(dw) as new_rows:
        q_idx = _project(dw, D_MODEL, with_kv=False, inputs=p)
        for dev, ref in ((_u16(q_idx), O.round_bf16_bits(O.index_projection(h, wq))),
                         (_u16(dw.k_idx[new_rows]), O.round_bf16_bits(O.index_projection(h, wk)))):
            # same sign, adjacent bit patterns: at most one unit in the last place apart
            d = np.abs(dev.astype(np.int32) - ref.astype(np.int32))
            assert np.all((d <= 1) & ((dev >> 15) == (ref >> 15)))
            assert np.mean(d == 0) >= 0.95, np.mean(d == 0)
            _say(f"normal inputs: {np.mean(d == 0):.4f} exact, {np.sum(d == 1)} one ulp apart")


@pytest.mark.parametrize("cfg,check", [(1, None), (2, [0, 7]), (3, [3, 15]), (5, [0, 33, 63])])
def test_step_after_projection_vs_oracle(cfg, check):
    """The decode step of a token that has just been appended: its projected indexer query scores
    the cache that now holds its projected indexer key and its K/V rows."""
    w = cs.config(cfg)
    dw = device_workload(w)
    dims, rows = dims_of(dw), rows_of(dw)
    ws, nws = workspace(dims, rows)
    R = w.n_rows
    with _restored_new_rows(dw):
        q_idx = _project(dw, D_MODEL)
        out = torch.zeros((R, w.n_layers, w.hq, 128), dtype=torch.int16, device="cuda")
        idx = torch.full((R, w.topk), -7, dtype=torch.int32, device="cuda")
        cnt = torch.full((R,), -7, dtype=torch.int32, device="cuda")
        clsa.step(dims, rows, q_idx, dw.k_idx, dw.k_cache, dw.v_cache, dw.cu_seqlens, dw.q, out, idx, cnt, ws, nws)
        torch.cuda.synchronize()
        idx_h, cnt_h, dev = idx.cpu().numpy(), cnt.cpu().numpy(), bf16_dev_to_f64(out)
    n_new_selected = 0
    for r in (range(R) if check is None else check):
        ref = oracle_row_projected(w, r, D_MODEL)
        assert cnt_h[r] == ref["count"]
        assert np.array_equal(idx_h[r], ref["idx"]), f"cfg{cfg} row {r}: {np.sum(idx_h[r] != ref['idx'])} mismatches"
        n_new_selected += int(w.row_len(r) - 1 in ref["sel"])
        st = assert_outputs_close(dev[r], ref["out"], f"projected cfg{cfg} row {r}")
        _say(f"projected step cfg{cfg} row {r}: max {st[0]:.2e} mean {st[1]:.2e} rel {st[2]:.2e}")
    _say(f"cfg{cfg}: new token selected in {n_new_selected} checked rows")
