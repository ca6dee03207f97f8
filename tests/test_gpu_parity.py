"""Parity of the HIP path (through the C ABI) with the fp64 CPU oracle, on the five workloads
and on edge cases.  Indices and scores must match bit for bit; attention outputs within the
tolerance in _gpu_helpers (max-abs 2e-2, mean-abs 2e-3, relative Frobenius 5e-3)."""
import zlib

import numpy as np
import pytest
import torch

import clsa_synth as cs
import cross_layer_token_amd as clsa
from _gpu_helpers import (assert_outputs_close, bf16_dev_to_f64, cu_tensor, device_workload, dims_of, rows_of,
                          workspace)
from clsa_synth import gen
from oracle import clsa_oracle as O
from oracle.workload_oracle import oracle_row

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    yield
    torch.cuda.synchronize()


def _say(*a):
    print(*a, flush=True)


# ----------------------------------------------------------------------------- generator
@pytest.mark.parametrize("cfg", [1, 3])
def test_device_generator_matches_host(cfg):
    w = cs.config(cfg)
    dw = device_workload(w)
    rng = np.random.default_rng(cfg)
    T = w.total_tokens
    toks = np.unique(np.concatenate([rng.integers(0, T, 300), [t for t, _ in w.needle_pairs()][:64], [0, T - 1]]))
    assert np.array_equal(dw.k_idx[torch.from_numpy(toks).cuda()].cpu().numpy().view(np.uint16), w.k_idx_bits(toks))
    assert np.array_equal(dw.q_idx.cpu().numpy().view(np.uint16), w.q_idx_bits(np.arange(w.n_rows)))
    for which, t in (("k", dw.k_cache), ("v", dw.v_cache)):
        got = t[torch.from_numpy(toks).cuda()].cpu().numpy().view(np.uint16)
        assert np.array_equal(got, w.kv_bits(toks, which))
    rows = np.array([0, w.n_rows - 1])
    assert np.array_equal(dw.q[torch.from_numpy(rows).cuda()].cpu().numpy().view(np.uint16), w.q_bits(rows))


# ----------------------------------------------------------------------------- a1 scores
def _decode_scores(dw):
    w = dw.w
    dims, rows = dims_of(dw), rows_of(dw)
    ld = ((w.max_row_len + 63) // 64) * 64
    scores = torch.full((w.n_rows, ld), float("nan"), dtype=torch.float32, device="cuda")
    clsa.index_scores(dims, rows, dw.q_idx, dw.k_idx, dw.cu_seqlens, scores, ld)
    torch.cuda.synchronize()
    return scores


@pytest.mark.parametrize("cfg,check_rows", [(1, None), (2, None), (3, [0, 15]), (5, [0, 1, 17, 63])])
def test_index_scores_decode_bitwise(cfg, check_rows):
    w = cs.config(cfg)
    dw = device_workload(w)
    scores = _decode_scores(dw)
    cu = w.cu_seqlens
    for r in (range(w.n_rows) if check_rows is None else check_rows):
        n = w.row_len(r)
        ref = O.index_scores(w.q_idx_f64([r])[0], w.k_idx_f64(cu[r] + np.arange(n)))
        got = scores[r, :n].cpu().numpy().astype(np.float64)
        assert np.array_equal(got, ref), f"cfg{cfg} row {r}: {np.sum(got != ref)} mismatches"
    _say(f"cfg{cfg} scores bitwise OK")


def _prefill_scores_check(w, dw, pos0, m, ld):
    """clsa_index_scores on prefill rows pos0 .. pos0 + m - 1 of sequence 0: every row bitwise
    against the oracle's scores of its visible tokens, and nothing written above the diagonal."""
    sc = torch.full((m, ld), float("nan"), dtype=torch.float32, device="cuda")
    clsa.index_scores(dims_of(dw), rows_of(dw, row0=pos0, n_rows=m), dw.q_idx[pos0:], dw.k_idx, dw.cu_seqlens, sc, ld)
    torch.cuda.synchronize()
    cols = torch.arange(ld, device="cuda")[None, :]
    lim = pos0 + torch.arange(m, device="cuda")[:, None]
    assert torch.isnan(sc.masked_fill(cols <= lim, float("nan"))).all(), "wrote above the causal diagonal"
    assert not torch.isnan(sc.masked_fill(cols > lim, 0.0)).any(), "left a visible entry unwritten"
    host = sc.cpu().numpy()
    kf = w.k_idx_f64(np.arange(pos0 + m))
    qf = w.q_idx_f64(np.arange(pos0, pos0 + m))
    for i in range(m):
        t = pos0 + i
        ref = O.index_scores(qf[i], kf[: t + 1])
        got = host[i, : t + 1].astype(np.float64)
        assert np.array_equal(got, ref), f"row {t}: {np.sum(got != ref)} mismatches"


def test_index_scores_prefill_bitwise():
    """The causal indexer GEMM on the 8192-row prefill workload in one call: every row bitwise
    against the oracle, nothing written above the diagonal; then calls that start mid-sequence at
    offsets that are not multiples of the 128-row tile."""
    w = cs.config(4)
    dw = device_workload(w, with_kv=False, with_q=False)
    _prefill_scores_check(w, dw, 0, w.n_rows, w.n_rows)
    _say("prefill scores: all 8192 rows bitwise")
    for pos0, m, ld in ((3000, 200, 3200), (50, 700, 752), (8000, 192, 8192), (127, 1, 128)):
        _prefill_scores_check(w, dw, pos0, m, ld)


def test_index_scores_prefill_d64_bitwise():
    w = cs.custom(mode="prefill", seq_lens=(1500,), d_idx=64, topk=64, n_layers=1, hq=4, hkv=1, needles=3, seed=57,
                  name="prefill_scores_d64")
    dw = device_workload(w, with_kv=False, with_q=False)
    _prefill_scores_check(w, dw, 0, 1500, 1536)
    _prefill_scores_check(w, dw, 333, 1000, 1336)


# ----------------------------------------------------------------------------- a2 top-k
def _score_rows(kind, lengths, rng):
    out = []
    for n in lengths:
        if kind == "ties":
            s = rng.integers(-3, 4, n).astype(np.float32) * 0.5
        elif kind == "normal":
            s = rng.standard_normal(n).astype(np.float32) * 4
        elif kind == "equal":
            s = np.full(n, 1.25, dtype=np.float32)
        elif kind == "zeros":
            s = np.where(rng.integers(0, 2, n) == 1, np.float32(0.0), np.float32(-0.0)).astype(np.float32)
            s[rng.integers(0, n, max(1, n // 100))] = 1.0
        else:  # quantised to 1/16 in [-8, 8], like the ragged workload
            s = (rng.integers(-128, 129, n) / 16.0).astype(np.float32)
        out.append(s)
    return out


def _run_topk_decode(rows_scores, k):
    lengths = [len(s) for s in rows_scores]
    B = len(lengths)
    ld = ((max(lengths) + 63) // 64) * 64
    host = np.full((B, ld), np.nan, dtype=np.float32)
    for i, s in enumerate(rows_scores):
        host[i, : len(s)] = s
    dims = clsa.make_dims(B, 128, k, 1, 8, 2)
    cu = np.concatenate([[0], np.cumsum(lengths)])
    rows = clsa.make_rows(clsa.MODE_DECODE, B, max(lengths), int(cu[-1]), cu_seqlens_host=cu.tolist())
    ws, nws = workspace(dims, rows)
    idx = torch.full((B, k), -7, dtype=torch.int32, device="cuda")
    cnt = torch.full((B,), -7, dtype=torch.int32, device="cuda")
    clsa.topk(dims, rows, cu_tensor(lengths), torch.from_numpy(host).cuda(), ld, idx, cnt, ws, nws)
    torch.cuda.synchronize()
    return idx.cpu().numpy(), cnt.cpu().numpy()


SHORT_ROWS = [1, 5, 300, 2048, 4096, 12288]                       # one workgroup per row (LDS)
LONG_ROWS = [1, 5, 300, 2048, 4096, 12288, 12289, 50000, 131072]   # histogram select over many workgroups


@pytest.mark.parametrize("lengths", [SHORT_ROWS, LONG_ROWS], ids=["short", "long"])
@pytest.mark.parametrize("kind", ["ties", "normal", "equal", "zeros", "q16"])
@pytest.mark.parametrize("k", [1, 7, 256, 2048])
def test_topk_matches_oracle_on_given_scores(kind, k, lengths):
    rng = np.random.default_rng(zlib.crc32(f"{kind}-{k}-{len(lengths)}".encode()))
    rs = _score_rows(kind, lengths, rng)
    idx, cnt = _run_topk_decode(rs, k)
    for i, s in enumerate(rs):
        sel = O.topk_select(s.astype(np.float64), k)
        want, m = O.pad_selection(sel, k)
        assert cnt[i] == m, (kind, k, lengths[i])
        assert np.array_equal(idx[i], want), f"{kind} k={k} n={lengths[i]}: {np.sum(idx[i] != want)} mismatches"


@pytest.mark.parametrize("kind,k", [("ties", 65536), ("normal", 2048)])
def test_topk_at_the_maximum_row_length(kind, k):
    """One row of CLSA_MAX_ROW_LEN = 2^24 scores (2048 select spans, the most a row has), at the
    largest k (65536: the candidate list far exceeds LDS and is refined in the workspace) and at
    the 128K workload's k."""
    n = 1 << 24
    rng = np.random.default_rng(61 if kind == "ties" else 62)
    s = _score_rows(kind, [n], rng)[0]
    idx, cnt = _run_topk_decode([s], k)
    want, m = O.pad_selection(O.topk_select(s.astype(np.float64), k), k)
    assert cnt[0] == m and np.array_equal(idx[0], want), f"{np.sum(idx[0] != want)} mismatches"


def test_sparse_attn_reads_cache_rows_past_2_to_the_32_elements():
    """A 5M-token sequence with 8 KV heads: a cache row is hkv * 128 = 1024 elements, so every
    token from 2^22 on lies more than 2^32 elements into the cache.  Attention over 1024 selected
    tokens spread over the whole sequence (about a sixth of them past 2^22), read from the cache
    and from the gathered compact buffer, against the oracle."""
    n, k = 5_000_000, 1024
    w = cs.custom(seq_lens=(n,), d_idx=64, topk=k, n_layers=2, hq=16, hkv=8, seed=71, name="long_cache")
    dw = device_workload(w)
    sel = np.sort(np.random.default_rng(71).choice(n, k, replace=False))
    assert (sel >= (1 << 22)).sum() > 100
    idx = torch.from_numpy(sel.astype(np.int32)[None, :]).cuda()
    cnt = torch.tensor([k], dtype=torch.int32, device="cuda")
    kf, vf = w.kv_f64(sel)                       # sequence 0 starts at cache row 0
    ref = O.sparse_attention(w.q_f64([0])[0], kf, vf)
    dims, rows = dims_of(dw), rows_of(dw)
    L, hq = w.n_layers, w.hq
    row_el = L * hq * 128
    ws, nws = workspace(dims, rows, clsa.SCHEDULE_PER_LAYER)
    ksel = torch.empty((1, w.hkv, k, 128), dtype=torch.int16, device="cuda")
    vsel = torch.empty_like(ksel)
    clsa.gather_kv(dims, rows, dw.k_cache, dw.v_cache, dw.cu_seqlens, idx, cnt, ksel, vsel)
    for src in ("cache", "compact"):
        out = torch.zeros((1, L, hq, 128), dtype=torch.int16, device="cuda")
        ks_, vs_ = (ksel, vsel) if src == "compact" else (None, None)
        clsa.sparse_attn(dims, rows, dw.q, row_el, L, ks_, vs_, dw.k_cache, dw.v_cache, dw.cu_seqlens, idx, cnt, out,
                         row_el, ws, nws)
        torch.cuda.synchronize()
        assert_outputs_close(bf16_dev_to_f64(out)[0], ref, f"5M-token cache, {src}")


def test_topk_prefill_rows_lds_path():
    rng = np.random.default_rng(5)
    n, k = 3000, 256
    s = (rng.integers(-40, 41, (n, n)) / 8.0).astype(np.float32)
    dims = clsa.make_dims(1, 128, k, 1, 8, 2)
    rows = clsa.make_rows(clsa.MODE_PREFILL, n, n, n, seq=0, pos0=0, cu_seqlens_host=[0, n])
    idx = torch.empty((n, k), dtype=torch.int32, device="cuda")
    cnt = torch.empty((n,), dtype=torch.int32, device="cuda")
    ws, nws = workspace(dims, rows)
    clsa.topk(dims, rows, cu_tensor([n]), torch.from_numpy(s).cuda(), n, idx, cnt, ws, nws)
    torch.cuda.synchronize()
    idx, cnt = idx.cpu().numpy(), cnt.cpu().numpy()
    for t in list(range(0, 300)) + [1000, 2999]:
        want, m = O.pad_selection(O.topk_select(s[t, : t + 1].astype(np.float64), k), k)
        assert cnt[t] == m and np.array_equal(idx[t], want), t


# ----------------------------------------------------------------------------- a3 gather, a4 attention
def _oracle_idx(w, rows):
    res = [oracle_row(w, r) for r in rows]
    return res


@pytest.mark.parametrize("cfg", [1, 2])
def test_gather_and_attention_on_oracle_selection(cfg):
    w = cs.config(cfg)
    dw = device_workload(w)
    res = _oracle_idx(w, range(w.n_rows))
    idx = torch.from_numpy(np.stack([r["idx"] for r in res])).cuda()
    cnt = torch.from_numpy(np.array([r["count"] for r in res], dtype=np.int32)).cuda()
    dims, rows = dims_of(dw), rows_of(dw)
    R, k = w.n_rows, w.topk
    ksel = torch.empty((R, w.hkv, k, 128), dtype=torch.int16, device="cuda")
    vsel = torch.empty_like(ksel)
    clsa.gather_kv(dims, rows, dw.k_cache, dw.v_cache, dw.cu_seqlens, idx, cnt, ksel, vsel)
    torch.cuda.synchronize()
    cu = w.cu_seqlens
    for r in range(R):
        m = res[r]["count"]
        toks = cu[r] + res[r]["sel"]
        assert np.array_equal(ksel[r, :, :m].permute(1, 0, 2).cpu().numpy().view(np.uint16), w.kv_bits(toks, "k"))
        assert np.array_equal(vsel[r, :, :m].permute(1, 0, 2).cpu().numpy().view(np.uint16), w.kv_bits(toks, "v"))
        assert not ksel[r, :, m:].any() and not vsel[r, :, m:].any()
    ref = np.stack([r["out"] for r in res])
    L, hq = w.n_layers, w.hq
    row_el = L * hq * 128
    ws, nws = workspace(dims, rows, clsa.SCHEDULE_PER_LAYER)
    for src in ("compact", "cache"):
        out = torch.zeros((R, L, hq, 128), dtype=torch.int16, device="cuda")
        ks_, vs_ = (ksel, vsel) if src == "compact" else (None, None)
        clsa.sparse_attn(dims, rows, dw.q, row_el, L, ks_, vs_, dw.k_cache, dw.v_cache, dw.cu_seqlens, idx, cnt, out,
                         row_el, ws, nws)
        torch.cuda.synchronize()
        st = assert_outputs_close(bf16_dev_to_f64(out), ref, f"cfg{cfg} {src} all layers")
        _say(f"cfg{cfg} attention {src} L-batched", st)
        out.zero_()
        for layer in range(L):   # one layer per call, strided rows
            clsa.sparse_attn(dims, rows, dw.q[:, layer], row_el, 1, ks_, vs_, dw.k_cache, dw.v_cache, dw.cu_seqlens,
                             idx, cnt, out[:, layer], row_el, ws, nws)
        torch.cuda.synchronize()
        assert_outputs_close(bf16_dev_to_f64(out), ref, f"cfg{cfg} {src} per layer")


def test_attention_paired_kv_heads():
    """Many (row, KV head) blocks of 33-64 query rows (256 rows x 2 KV heads, 3 layers x 12 heads
    per KV head = 36 query rows) run one eight-wave workgroup per (row, pair of KV heads), a team
    per head.  The oracle's selections read through idx from the cache and from the gathered
    compact buffers, every row against the oracle."""
    rng = np.random.default_rng(5)
    lens = tuple(int(x) for x in rng.integers(150, 900, 256))
    w = cs.custom(seq_lens=lens, d_idx=64, topk=128, n_layers=3, hq=24, hkv=2, needles=1, seed=73,
                  name="paired_heads")
    dw = device_workload(w)
    res = _oracle_idx(w, range(w.n_rows))
    R, k, L, hq = w.n_rows, w.topk, w.n_layers, w.hq
    idx = torch.from_numpy(np.stack([x["idx"] for x in res])).cuda()
    cnt = torch.from_numpy(np.array([x["count"] for x in res], dtype=np.int32)).cuda()
    dims, rows = dims_of(dw), rows_of(dw)
    ksel = torch.empty((R, w.hkv, k, 128), dtype=torch.int16, device="cuda")
    vsel = torch.empty_like(ksel)
    clsa.gather_kv(dims, rows, dw.k_cache, dw.v_cache, dw.cu_seqlens, idx, cnt, ksel, vsel)
    row_el = L * hq * 128
    ws, nws = workspace(dims, rows, clsa.SCHEDULE_PER_LAYER)
    ref = np.stack([x["out"] for x in res])
    for src in ("cache", "compact"):
        out = torch.zeros((R, L, hq, 128), dtype=torch.int16, device="cuda")
        ks_, vs_ = (ksel, vsel) if src == "compact" else (None, None)
        clsa.sparse_attn(dims, rows, dw.q, row_el, L, ks_, vs_, dw.k_cache, dw.v_cache, dw.cu_seqlens, idx, cnt, out,
                         row_el, ws, nws)
        torch.cuda.synchronize()
        st = assert_outputs_close(bf16_dev_to_f64(out), ref, f"paired heads, {src}")
        _say(f"paired heads from {src}: {R} rows", st)


@pytest.mark.parametrize("counts", [[1, 2, 63, 64, 65, 100], [5, 5, 5, 5, 5, 5]])
def test_attention_ragged_counts_and_splits(counts):
    """Short selections (count < k), single-row selections, tiles with a ragged tail."""
    w = cs.custom(seq_lens=(700, 300, 128, 90, 1000, 256), topk=100, n_layers=3, hq=8, hkv=2, seed=21)
    dw = device_workload(w)
    rng = np.random.default_rng(3)
    k = w.topk
    idx_h = np.full((w.batch, k), -1, dtype=np.int32)
    sels = []
    for b, c in enumerate(counts):
        sel = np.sort(rng.choice(w.seq_lens[b], size=c, replace=False))
        idx_h[b, :c] = sel
        sels.append(sel)
    idx = torch.from_numpy(idx_h).cuda()
    cnt = torch.tensor(counts, dtype=torch.int32, device="cuda")
    dims, rows = dims_of(dw), rows_of(dw)
    L, hq = w.n_layers, w.hq
    row_el = L * hq * 128
    out = torch.zeros((w.batch, L, hq, 128), dtype=torch.int16, device="cuda")
    ws, nws = workspace(dims, rows)
    clsa.sparse_attn(dims, rows, dw.q, row_el, L, None, None, dw.k_cache, dw.v_cache, dw.cu_seqlens, idx, cnt, out,
                     row_el, ws, nws)
    torch.cuda.synchronize()
    cu = w.cu_seqlens
    dev = bf16_dev_to_f64(out)
    for b in range(w.batch):
        kf, vf = w.kv_f64(cu[b] + sels[b])
        ref = O.sparse_attention(w.q_f64([b])[0], kf, vf)
        assert_outputs_close(dev[b], ref, f"row {b} count {counts[b]}")
        if counts[b] == 1:   # one selected row: every head returns that V row (bf16 exact)
            for h in range(hq):
                assert np.array_equal(dev[b, :, h], np.broadcast_to(vf[0, h // (hq // w.hkv)], (L, 128)))


# ----------------------------------------------------------------------------- whole step
_CPP_CACHE: dict = {}


def _oracle_threads() -> int:
    import os
    return max(1, min(16, os.cpu_count() or 1))


def _cpp_rows(w, rows, routing=False):
    """The C++ fp64 oracle (its own input generator) on the given rows over the host's threads,
    each row single-threaded; cached per workload, rows and kind, so both schedules compare
    against one evaluation."""
    from oracle import cpp as C
    key = (w.name, w.seed, tuple(int(r) for r in rows), routing)
    if key not in _CPP_CACHE:
        f = C.oracle_rows_layer_routing if routing else C.oracle_rows
        _CPP_CACHE[key] = f(w, list(rows), threads=_oracle_threads())
    return _CPP_CACHE[key]


def _run_step(dw, schedule, rows_kw=None, chunk=0, want_scores=False):
    w = dw.w
    dims = dims_of(dw)
    rows = rows_of(dw, **(rows_kw or {}))
    R = rows.n_rows
    ws, nws = workspace(dims, rows, schedule, chunk)
    out = torch.zeros((R, w.n_layers, w.hq, 128), dtype=torch.int16, device="cuda")
    idx = torch.full((R, w.topk), -7, dtype=torch.int32, device="cuda")
    cnt = torch.full((R,), -7, dtype=torch.int32, device="cuda")
    row0 = (rows_kw or {}).get("row0", 0)
    clsa.step(dims, rows, dw.q_idx[row0:], dw.k_idx, dw.k_cache, dw.v_cache, dw.cu_seqlens, dw.q[row0:], out, idx, cnt,
              ws, nws, schedule=schedule, prefill_chunk_rows=chunk)
    torch.cuda.synchronize()
    return idx.cpu().numpy(), cnt.cpu().numpy(), out


@pytest.mark.parametrize("cfg,check", [(1, None), (2, None), (3, [0, 7, 15]), (5, [0, 5, 31, 63])])
@pytest.mark.parametrize("schedule", [clsa.SCHEDULE_LAYER_BATCHED, clsa.SCHEDULE_PER_LAYER])
def test_step_decode_vs_oracle(cfg, check, schedule):
    """Every row of the workload against the threaded C++ oracle (selections bitwise, outputs
    within the tolerance), and the listed rows (all rows of the two small workloads) against the
    numpy oracle as well, with its needle check."""
    w = cs.config(cfg)
    dw = device_workload(w)
    idx, cnt, out = _run_step(dw, schedule)
    dev = bf16_dev_to_f64(out)
    ref_all = _cpp_rows(w, range(w.n_rows))
    worst = np.zeros(3)
    for r in range(w.n_rows):
        assert cnt[r] == ref_all["count"][r], f"cfg{cfg} row {r}: count"
        assert np.array_equal(idx[r], ref_all["idx"][r]), \
            f"cfg{cfg} row {r}: {np.sum(idx[r] != ref_all['idx'][r])} index mismatches (C++ oracle)"
        worst = np.maximum(worst, assert_outputs_close(dev[r], ref_all["out"][r], f"cfg{cfg} row {r} (C++ oracle)"))
    _say(f"cfg{cfg} sched {schedule}: all {w.n_rows} rows vs the C++ oracle, worst max {worst[0]:.2e} "
         f"mean {worst[1]:.2e} rel {worst[2]:.2e}")
    rows = range(w.n_rows) if check is None else check
    for r in rows:
        res = oracle_row(w, r)
        assert cnt[r] == res["count"]
        assert np.array_equal(idx[r], res["idx"]), f"cfg{cfg} row {r}: {np.sum(idx[r] != res['idx'])} index mismatches"
        assert set(w.needle_positions_of_row(r)) <= set(idx[r].tolist())
        st = assert_outputs_close(dev[r], res["out"], f"cfg{cfg} row {r}")
        _say(f"cfg{cfg} sched {schedule} row {r}: max {st[0]:.2e} mean {st[1]:.2e} rel {st[2]:.2e}")
    # every row: count and structure (ascending, in range, -1 padded)
    for r in range(w.n_rows):
        m = min(w.topk, w.row_len(r))
        assert cnt[r] == m
        assert np.all(np.diff(idx[r, :m]) > 0) and idx[r, 0] >= 0 and idx[r, m - 1] < w.row_len(r)
        assert np.all(idx[r, m:] == -1)


@pytest.mark.parametrize("schedule", [clsa.SCHEDULE_LAYER_BATCHED, clsa.SCHEDULE_PER_LAYER])
def test_step_decode_mixed_lengths_vs_cpp_oracle(schedule):
    """One batch mixing a single-token row, rows shorter than k, exactly k and k + 1 tokens, and a
    row long enough that the select's last workgroup walks more than 16 span lists; every row
    against the independent C++ oracle."""
    from oracle import cpp as C
    w = cs.custom(seq_lens=(1, 100, 2047, 2048, 2049, 12289, 200000), d_idx=128, topk=2048, n_layers=3, hq=8, hkv=2,
                  needles=0, seed=77, name="mixed_lengths")
    dw = device_workload(w)
    idx, cnt, out = _run_step(dw, schedule)
    dev = bf16_dev_to_f64(out)
    for r in range(w.n_rows):
        res = C.oracle_row(w, r)
        assert cnt[r] == res["count"] == min(w.topk, w.row_len(r)), r
        assert np.array_equal(idx[r], res["idx"]), f"row {r}: {np.sum(idx[r] != res['idx'])} index mismatches"
        st = assert_outputs_close(dev[r], res["out"], f"mixed row {r}")
        _say(f"mixed sched {schedule} row {r} (n={w.row_len(r)}): max {st[0]:.2e} mean {st[1]:.2e} rel {st[2]:.2e}")


@pytest.mark.parametrize("lo,hi,den", [(-1, 1, 4), (0, 0, 1)], ids=["ties", "all_equal"])
def test_step_decode_heavy_ties_long_rows(lo, hi, den):
    """Long rows with tie-heavy scores.  Indexer entries {-1, 0, 1} / 4: a few thousand candidates
    around the k-th score, many of them tied.  All entries 0: every score ties, every token is a
    candidate - more than a workgroup keeps in LDS - and the selection (the lowest k tokens) is
    finished from the span lists in place.  Every row against the oracle."""
    w = cs.custom(seq_lens=(60000, 45000, 70001, 52000), d_idx=128, topk=2048, n_layers=4, hq=16, hkv=4, idx_lo=lo,
                  idx_hi=hi, idx_den=den, needles=0, seed=41, name=f"ties_long_{lo}_{hi}")
    dw = device_workload(w)
    for schedule in (clsa.SCHEDULE_LAYER_BATCHED, clsa.SCHEDULE_PER_LAYER):
        idx, cnt, out = _run_step(dw, schedule)
        dev = bf16_dev_to_f64(out)
        for r in range(w.n_rows):
            res = oracle_row(w, r)
            assert cnt[r] == res["count"]
            assert np.array_equal(idx[r], res["idx"]), f"row {r}: {np.sum(idx[r] != res['idx'])} index mismatches"
            assert_outputs_close(dev[r], res["out"], f"heavy ties row {r}")
        _say(f"heavy ties, schedule {schedule}: {w.n_rows} rows match")


def test_step_decode_segments_spanning_several_sequences():
    """The decode score kernel cuts the sequences' concatenated tokens into equal segments (1024
    tokens here), so a segment can hold the end of one sequence, whole short sequences and the
    start of the next.  Sequences at or below k (all taken), just above k (a partial in each of
    two segments) and long ones, mixed: every row against the oracle, both schedules."""
    lens = (13000, 300, 700, 1500, 90, 2100, 20000, 640, 999, 14000)
    w = cs.custom(seq_lens=lens, d_idx=128, topk=512, n_layers=2, hq=8, hkv=2, needles=2, seed=71,
                  name="segments_across_sequences")
    dw = device_workload(w)
    for schedule in (clsa.SCHEDULE_LAYER_BATCHED, clsa.SCHEDULE_PER_LAYER):
        idx, cnt, out = _run_step(dw, schedule)
        dev = bf16_dev_to_f64(out)
        for r in range(w.n_rows):
            res = oracle_row(w, r)
            assert cnt[r] == res["count"]
            assert np.array_equal(idx[r], res["idx"]), f"row {r}: {np.sum(idx[r] != res['idx'])} index mismatches"
            assert_outputs_close(dev[r], res["out"], f"segments across sequences row {r}")
        _say(f"segments across sequences, schedule {schedule}: {w.n_rows} rows match")


def test_step_decode_segments_holding_hundreds_of_short_sequences():
    """One score-kernel segment can hold hundreds of short sequences (1 to 40 tokens here, all
    taken whole at k = 24 or cut to 24) between two long ones that need the multi-workgroup
    select: the workgroup walks every piece in order.  Sampled rows and every row's count and
    structure against the oracle, layer-batched schedule."""
    rng = np.random.default_rng(11)
    short = tuple(int(x) for x in rng.integers(1, 41, 300))
    lens = (14000,) + short + (13000,)
    w = cs.custom(seq_lens=lens, d_idx=64, topk=24, n_layers=2, hq=4, hkv=2, needles=1, seed=79,
                  name="hundreds_of_short_sequences")
    dw = device_workload(w)
    idx, cnt, out = _run_step(dw, clsa.SCHEDULE_LAYER_BATCHED)
    dev = bf16_dev_to_f64(out)
    check = [0, 1, 2, 57, 150, 299, 300, w.n_rows - 1]
    for r in check:
        res = oracle_row(w, r)
        assert cnt[r] == res["count"]
        assert np.array_equal(idx[r], res["idx"]), f"row {r}: {np.sum(idx[r] != res['idx'])} index mismatches"
        assert_outputs_close(dev[r], res["out"], f"short sequences row {r}")
    for r in range(w.n_rows):
        m = min(w.topk, w.row_len(r))
        assert cnt[r] == m
        row = idx[r]
        assert np.all(np.diff(row[:m]) > 0) and row[0] >= 0 and row[m - 1] < w.row_len(r) and np.all(row[m:] == -1)
    _say(f"hundreds of short sequences: {w.n_rows} rows, {len(check)} against the oracle")


def test_step_decode_k_near_the_median_of_a_chunk():
    """k = 490 against 1024-token chunks of tie-heavy scores ({-1, 0, 1} / 4 indexer entries, about
    485 positive scores per chunk): a chunk's 490th largest score is a small positive value or zero
    or below, so some chunks publish a window of their histogram and the others (the m-th largest
    far below their top bin) the whole histogram.  Every row against the oracle, both schedules."""
    w = cs.custom(seq_lens=(40000, 30000), d_idx=128, topk=490, n_layers=2, hq=8, hkv=2, idx_lo=-1, idx_hi=1,
                  idx_den=4, needles=3, seed=47, name="k_near_median")
    dw = device_workload(w)
    for schedule in (clsa.SCHEDULE_LAYER_BATCHED, clsa.SCHEDULE_PER_LAYER):
        idx, cnt, out = _run_step(dw, schedule)
        dev = bf16_dev_to_f64(out)
        for r in range(w.n_rows):
            res = oracle_row(w, r)
            assert cnt[r] == res["count"]
            assert np.array_equal(idx[r], res["idx"]), f"row {r}: {np.sum(idx[r] != res['idx'])} index mismatches"
            assert_outputs_close(dev[r], res["out"], f"k near median row {r}")
        _say(f"k near the chunk median, schedule {schedule}: {w.n_rows} rows match")


@pytest.mark.parametrize("lens,planted", [
    ((16000, 20000), ((0, 2048, 1024),)),
    ((200000, 150000), tuple((0, c * 1024, 100) for c in range(20)) + tuple((1, c * 1024 + 500, 100) for c in range(20))),
], ids=["one_chunk_lds", "twenty_chunks_in_place"])
def test_step_decode_chunk_holding_the_largest_keys(lens, planted):
    """The row's largest keys packed into a few stretches of tokens instead of spread over the
    row: needles fill one 1024-token stretch (the candidate lists of the spans are then very
    uneven), or twenty stretches of 100 tokens at 1024-token spacing in each of two long rows.
    Every row against the oracle, both schedules."""
    w = cs.custom(seq_lens=lens, d_idx=128, topk=2048, n_layers=2, hq=8, hkv=2, needles=0, seed=43,
                  name="packed_needles", planted=planted)
    dw = device_workload(w)
    for schedule in (clsa.SCHEDULE_LAYER_BATCHED, clsa.SCHEDULE_PER_LAYER):
        idx, cnt, out = _run_step(dw, schedule)
        dev = bf16_dev_to_f64(out)
        for r in range(w.n_rows):
            res = oracle_row(w, r)
            assert cnt[r] == res["count"]
            assert np.array_equal(idx[r], res["idx"]), f"row {r}: {np.sum(idx[r] != res['idx'])} index mismatches"
            assert set(w.needle_positions_of_row(r)) <= set(idx[r].tolist())
            assert_outputs_close(dev[r], res["out"], f"packed needles row {r}")
        _say(f"packed needles {lens}, schedule {schedule}: {w.n_rows} rows match")


def test_step_per_layer_chunks_with_caller_buffers():
    """The per-layer schedule gathers K_S/V_S a chunk of rows at a time (at most 192 MiB): at k = 65536
    with 8 KV heads a row's K_S/V_S alone is 256 MiB, so every row is its own chunk.  The caller's
    compact buffers and the workspace's give the same result bit for bit, and every row matches the
    C++ oracle."""
    w = cs.custom(seq_lens=(70000, 66000, 90000), d_idx=64, topk=65536, n_layers=2, hq=8, hkv=8, needles=2, seed=97,
                  name="per_layer_chunks")
    dw = device_workload(w)
    dims, rows = dims_of(dw), rows_of(dw)
    R, L, k = w.n_rows, w.n_layers, w.topk
    idx_a, cnt_a, out_a = _run_step(dw, clsa.SCHEDULE_PER_LAYER)
    ws, nws = workspace(dims, rows, clsa.SCHEDULE_PER_LAYER)
    ksel = torch.empty((R, w.hkv, k, 128), dtype=torch.int16, device="cuda")
    vsel = torch.empty_like(ksel)
    out = torch.zeros((R, L, w.hq, 128), dtype=torch.int16, device="cuda")
    idx = torch.full((R, k), -7, dtype=torch.int32, device="cuda")
    cnt = torch.full((R,), -7, dtype=torch.int32, device="cuda")
    clsa.step(dims, rows, dw.q_idx, dw.k_idx, dw.k_cache, dw.v_cache, dw.cu_seqlens, dw.q, out, idx, cnt, ws, nws,
              k_sel=ksel, v_sel=vsel, schedule=clsa.SCHEDULE_PER_LAYER)
    torch.cuda.synchronize()
    assert np.array_equal(idx.cpu().numpy(), idx_a) and torch.equal(out, out_a)
    ref = _cpp_rows(w, range(R))
    dev = bf16_dev_to_f64(out)
    for r in range(R):
        assert cnt_a[r] == ref["count"][r] and np.array_equal(idx_a[r], ref["idx"][r]), f"row {r}"
        assert_outputs_close(dev[r], ref["out"][r], f"per-layer chunk row {r}")
    # the caller's compact buffers hold each row's gathered K_S/V_S
    toks = w.cu_seqlens[2] + ref["idx"][2][: ref["count"][2]][:100]
    assert np.array_equal(ksel[2, :, :100].permute(1, 0, 2).cpu().numpy().view(np.uint16), w.kv_bits(toks, "k"))


def test_step_decode_several_query_blocks_per_kv_head():
    """128 query rows per KV head (8 layers x a GQA group of 16): two 64-row query blocks per
    (row, KV head), each with its own split partials and ticket, and one selection finished by the
    first block's first split.  Both schedules, every row against the C++ oracle."""
    w = cs.custom(seq_lens=(20000, 15000, 30000), d_idx=64, topk=512, n_layers=8, hq=32, hkv=2, needles=2, seed=79,
                  name="decode_qblocks")
    dw = device_workload(w)
    ref = _cpp_rows(w, range(w.n_rows))
    for schedule in (clsa.SCHEDULE_LAYER_BATCHED, clsa.SCHEDULE_PER_LAYER):
        idx, cnt, out = _run_step(dw, schedule)
        dev = bf16_dev_to_f64(out)
        for r in range(w.n_rows):
            assert cnt[r] == ref["count"][r] and np.array_equal(idx[r], ref["idx"][r]), f"schedule {schedule} row {r}"
            assert_outputs_close(dev[r], ref["out"][r], f"query blocks, schedule {schedule}, row {r}")


def test_step_decode_many_blocks_in_one_team():
    """1024 (row, KV head, query block) blocks of 64 query rows (128 rows x 4 KV heads x two
    blocks of a 128-row GQA group): four-wave workgroups, two per CU, one team each and no key
    split, since blocks with two query blocks per head do not pair KV heads.  Both schedules,
    every row against the C++ oracle."""
    w = cs.custom(seq_lens=tuple(700 + 13 * i for i in range(128)), d_idx=64, topk=256, n_layers=8, hq=64, hkv=4,
                  seed=83, name="decode_one_team")
    dw = device_workload(w)
    ref = _cpp_rows(w, range(w.n_rows))
    for schedule in (clsa.SCHEDULE_LAYER_BATCHED, clsa.SCHEDULE_PER_LAYER):
        idx, cnt, out = _run_step(dw, schedule)
        dev = bf16_dev_to_f64(out)
        for r in range(w.n_rows):
            assert cnt[r] == ref["count"][r] and np.array_equal(idx[r], ref["idx"][r]), f"schedule {schedule} row {r}"
            assert_outputs_close(dev[r], ref["out"][r], f"one team, schedule {schedule}, row {r}")


def test_step_decode_at_the_largest_k():
    """k = CLSA_MAX_TOPK = 65536 of a 100000-token row (one KV head, so one attention block split
    16 ways over 4096 keys each): selection and attention against the oracle, both schedules."""
    w = cs.custom(seq_lens=(100000,), d_idx=64, topk=65536, n_layers=2, hq=4, hkv=1, needles=4, seed=67,
                  name="largest_k")
    dw = device_workload(w)
    res = oracle_row(w, 0)
    for schedule in (clsa.SCHEDULE_LAYER_BATCHED, clsa.SCHEDULE_PER_LAYER):
        idx, cnt, out = _run_step(dw, schedule)
        assert cnt[0] == res["count"] == 65536
        assert np.array_equal(idx[0], res["idx"]), f"{np.sum(idx[0] != res['idx'])} index mismatches"
        assert_outputs_close(bf16_dev_to_f64(out)[0], res["out"], f"largest k, schedule {schedule}")


@pytest.mark.parametrize("cfg,check", [(1, None), (2, [0, 7]), (3, [4]), (5, [1])])
def test_step_per_layer_routing_vs_oracle(cfg, check):
    """The ablation without the shared index: every layer scores the cache with its own indexer
    query, selects its own set and attends over it (same kernels, once per layer).  Every row and
    layer against the threaded C++ oracle, the listed rows against the numpy oracle too."""
    from oracle.workload_oracle import oracle_row_layer_routing
    w = cs.config(cfg)
    dw = device_workload(w)
    lq = dw.layer_q_idx()
    host = gen.uniform_int_bf16(w.seed, gen.TID_Q_IDX_LAYER, np.arange(lq.numel()), w.idx_lo, w.idx_hi, w.idx_den)
    assert np.array_equal(lq.cpu().numpy().view(np.uint16).reshape(-1), host)   # device fill == host generator
    dims, rows = dims_of(dw), rows_of(dw)
    R, L, k = w.n_rows, w.n_layers, w.topk
    ws, nws = workspace(dims, rows, clsa.SCHEDULE_PER_LAYER_ROUTING)
    out = torch.zeros((R, L, w.hq, 128), dtype=torch.int16, device="cuda")
    idx = torch.full((L, R, k), -7, dtype=torch.int32, device="cuda")
    cnt = torch.full((L, R), -7, dtype=torch.int32, device="cuda")
    clsa.step(dims, rows, lq, dw.k_idx, dw.k_cache, dw.v_cache, dw.cu_seqlens, dw.q, out, idx, cnt, ws, nws,
              schedule=clsa.SCHEDULE_PER_LAYER_ROUTING)
    torch.cuda.synchronize()
    idx_h, cnt_h, dev = idx.cpu().numpy(), cnt.cpu().numpy(), bf16_dev_to_f64(out)
    ref_all = _cpp_rows(w, range(R), routing=True)
    for r in range(R):
        for l in range(L):
            assert cnt_h[l, r] == ref_all["count"][r, l], f"cfg{cfg} row {r} layer {l}: count"
            assert np.array_equal(idx_h[l, r], ref_all["idx"][r, l]), f"cfg{cfg} row {r} layer {l} (C++ oracle)"
        assert_outputs_close(dev[r], ref_all["out"][r], f"routing cfg{cfg} row {r} (C++ oracle)")
    _say(f"per-layer routing cfg{cfg}: all {R} rows x {L} layers vs the C++ oracle")
    for r in (range(R) if check is None else check):
        ref = oracle_row_layer_routing(w, r)
        for l in range(L):
            assert cnt_h[l, r] == ref["count"][l]
            assert np.array_equal(idx_h[l, r], ref["idx"][l]), f"cfg{cfg} row {r} layer {l}"
        assert_outputs_close(dev[r], ref["out"], f"routing cfg{cfg} row {r}")
    # the layers really route differently
    assert not np.array_equal(idx_h[0, 0], idx_h[1, 0])


def _prefill_sample(n, k):
    """Every 8th row, every row around k (where rows stop taking all their tokens) and the last 64."""
    return sorted(set(range(0, n, 8)) | set(range(k - 8, k + 9)) | set(range(n - 64, n)))


@pytest.mark.parametrize("schedule,chunk", [(clsa.SCHEDULE_LAYER_BATCHED, 8192), (clsa.SCHEDULE_LAYER_BATCHED, 1024),
                                            (clsa.SCHEDULE_PER_LAYER, 1024)])
def test_step_prefill_vs_oracle(schedule, chunk):
    """The 8192-row causal prefill, in one chunk of 8192 rows (the benchmark's) and in chunks of
    1024: every count, every 8th row, the rows around k and the last 64 rows against the threaded
    C++ oracle, and a few rows against the numpy oracle as well."""
    w = cs.config(4)
    dw = device_workload(w)
    idx, cnt, out = _run_step(dw, schedule, chunk=chunk)
    n = w.n_rows
    assert np.array_equal(cnt, np.minimum(np.arange(1, n + 1), w.topk))
    dev = bf16_dev_to_f64(out)
    sample = _prefill_sample(n, w.topk)
    ref_all = _cpp_rows(w, sample)
    for i, t in enumerate(sample):
        assert np.array_equal(idx[t], ref_all["idx"][i]), f"row {t}: {np.sum(idx[t] != ref_all['idx'][i])} mismatches"
        assert_outputs_close(dev[t], ref_all["out"][i], f"prefill row {t} (C++ oracle)")
    _say(f"prefill chunk {chunk} schedule {schedule}: {len(sample)} rows vs the C++ oracle")
    for t in [0, 1, 2, 100, 1023, 1024, 2046, 2047, 2048, 4095, 5000, 8191]:
        res = oracle_row(w, t)
        assert np.array_equal(idx[t], res["idx"]), f"row {t}"
        assert_outputs_close(dev[t], res["out"], f"prefill row {t}")
    assert set(w.needle_positions_of_row(n - 1)) <= set(idx[n - 1].tolist())


@pytest.mark.parametrize("n_layers,hq,hkv", [(2, 8, 2), (12, 16, 4)], ids=["8_query_rows", "48_query_rows"])
def test_step_prefill_query_rows_per_kv_head(n_layers, hq, hkv):
    """Prefill rows with 8 query rows per KV head (two teams of two waves, one of them with no
    query columns) and with 48 (one team of four waves, 64-row blocks): every 25th row and the
    k-boundary rows against the oracle, layer-batched."""
    w = cs.custom(mode="prefill", seq_lens=(1500,), d_idx=64, topk=256, n_layers=n_layers, hq=hq, hkv=hkv, seed=53,
                  name=f"prefill_q{n_layers * hq // hkv}")
    dw = device_workload(w)
    idx, cnt, out = _run_step(dw, clsa.SCHEDULE_LAYER_BATCHED, chunk=700)
    assert np.array_equal(cnt, np.minimum(np.arange(1, w.n_rows + 1), w.topk))
    dev = bf16_dev_to_f64(out)
    for t in sorted(set(range(0, w.n_rows, 25)) | {254, 255, 256, 257, w.n_rows - 1}):
        res = oracle_row(w, t)
        assert np.array_equal(idx[t], res["idx"]), f"row {t}"
        assert_outputs_close(dev[t], res["out"], f"prefill row {t}")


def test_step_prefill_chunking_invariance():
    w = cs.config(4)
    dw = device_workload(w)
    a = _run_step(dw, clsa.SCHEDULE_LAYER_BATCHED, chunk=1024)
    b = _run_step(dw, clsa.SCHEDULE_LAYER_BATCHED, chunk=300)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])
    assert torch.equal(a[2], b[2])
    # the same rows run as a call starting mid-sequence
    c = _run_step(dw, clsa.SCHEDULE_LAYER_BATCHED, rows_kw=dict(row0=5000, n_rows=1000), chunk=512)
    assert np.array_equal(a[0][5000:6000], c[0]) and torch.equal(a[2][5000:6000], c[2])


def test_step_prefill_selection_past_one_id_stage():
    """Prefill rows that select more tokens than the attention stages in LDS at a time (2048 ids):
    k = 5000 over a 6000-token sequence, so rows from 2048 on run the staged loop two or three
    times.  Rows around every stage boundary and the last rows against the C++ oracle."""
    w = cs.custom(mode="prefill", seq_lens=(6000,), d_idx=64, topk=5000, n_layers=2, hq=8, hkv=2, needles=3, seed=77,
                  name="prefill_k5000")
    dw = device_workload(w)
    idx, cnt, out = _run_step(dw, clsa.SCHEDULE_LAYER_BATCHED, chunk=1024)
    assert np.array_equal(cnt, np.minimum(np.arange(1, w.n_rows + 1), w.topk))
    rows = [0, 31, 2046, 2047, 2048, 2049, 2080, 4095, 4096, 4097, 4999, 5000, 5001, 5998, 5999]
    ref = _cpp_rows(w, rows)
    dev = bf16_dev_to_f64(out)
    for i, t in enumerate(rows):
        assert np.array_equal(idx[t], ref["idx"][i]), f"row {t}"
        assert_outputs_close(dev[t], ref["out"][i], f"prefill row {t}")


def test_step_prefill_rows_past_32bit_offsets():
    """The last rows of a prefill over a 2^20 + 2^18-token sequence with 8 KV heads: the rows a
    query row may select span more than 2^31 bytes of the cache from the sequence's base, so the
    prefill attention forms 64-bit row addresses instead of 32-bit buffer offsets.  Every row
    against the C++ oracle."""
    n = (1 << 20) + (1 << 18)
    w = cs.custom(mode="prefill", seq_lens=(n,), d_idx=64, topk=512, n_layers=1, hq=8, hkv=8, needles=2, seed=71,
                  name="prefill_past_32bit")
    assert n * w.hkv * 128 * 2 > 2**31 - 1
    dw = device_workload(w)
    rows = list(range(n - 6, n))
    idx, cnt, out = _run_step(dw, clsa.SCHEDULE_LAYER_BATCHED, rows_kw=dict(row0=rows[0], n_rows=len(rows)), chunk=8)
    ref = _cpp_rows(w, rows)
    dev = bf16_dev_to_f64(out)
    for i, t in enumerate(rows):
        assert cnt[i] == ref["count"][i] == w.topk
        assert np.array_equal(idx[i], ref["idx"][i]), f"row {t}"
        assert_outputs_close(dev[i], ref["out"][i], f"prefill row {t}")
    # the selections reach past the first 2^31 bytes of the head's rows
    assert max(int(idx[i].max()) for i in range(len(rows))) * w.hkv * 256 > 2**31


def test_step_is_deterministic():
    w = cs.config(2)
    dw = device_workload(w)
    a = _run_step(dw, clsa.SCHEDULE_LAYER_BATCHED)
    b = _run_step(dw, clsa.SCHEDULE_LAYER_BATCHED)
    assert np.array_equal(a[0], b[0]) and torch.equal(a[2], b[2])


def test_step_k_at_least_n_is_dense_attention():
    w = cs.custom(seq_lens=(200, 77, 513), topk=600, n_layers=2, hq=8, hkv=2, seed=31)
    dw = device_workload(w)
    idx, cnt, out = _run_step(dw, clsa.SCHEDULE_LAYER_BATCHED)
    dev = bf16_dev_to_f64(out)
    cu = w.cu_seqlens
    for b, n in enumerate(w.seq_lens):
        assert cnt[b] == n and np.array_equal(idx[b, :n], np.arange(n))
        kf, vf = w.kv_f64(cu[b] + np.arange(n))
        assert_outputs_close(dev[b], O.sparse_attention(w.q_f64([b])[0], kf, vf), f"dense row {b}")


# ---- seeded random shapes ---------------------------------------------------------------------
# Shapes drawn once from a fixed seed, so the cases are the same on every run.  k and the
# (query head, KV head) counts cycle through their lists (every value appears); batch sizes,
# sequence lengths from 1 token to tens of thousands (some exactly k - 1, k or k + 1), 1 to 6
# layers, both indexer widths and the needles are drawn; every third decode shape has tie-heavy
# indexer values and every fifth one sequence of 100K-140K tokens.  They reach the plan's choices (one or two
# teams, paired KV heads, 1 to 16 splits, the fused or separate selection, the LDS or span-list
# top-k) in combinations the named cases above do not.
_HEADS = [(4, 4), (8, 2), (16, 4), (32, 8), (12, 3), (6, 1), (8, 8), (2, 1)]
_KS = [1, 7, 100, 512, 1500, 2048, 3000]


def _decode_draws(n=20, seed=2024):
    rng = np.random.default_rng(seed)
    draws = []
    for i in range(n):
        k = _KS[i % len(_KS)]
        b = int(rng.integers(1, 17))
        lens = [max(1, int(np.exp(rng.uniform(0.0, np.log(30000))))) for _ in range(b)]
        for j in range(b):
            if rng.random() < 0.2:
                lens[j] = max(1, k + int(rng.integers(-1, 2)))
        if i % 5 == 4:  # one long sequence: the multi-workgroup select over many spans
            lens[0] = int(rng.integers(100000, 140001))
        hq, hkv = _HEADS[i % len(_HEADS)]
        ties = i % 3 == 0
        draws.append(dict(seq_lens=tuple(lens), topk=k, n_layers=int(rng.integers(1, 7)), hq=hq, hkv=hkv,
                          d_idx=int(rng.choice([64, 128])), needles=int(rng.choice([0, 2])) if min(lens) >= 2 else 0,
                          idx_lo=-1 if ties else -8, idx_hi=1 if ties else 8, idx_den=4 if ties else 8,
                          seed=1000 + i, name=f"random_decode_{i}"))
    return draws


def _prefill_draws(n=10, seed=4096):
    rng = np.random.default_rng(seed)
    draws = []
    for i in range(n):
        length = int(rng.integers(50, 1201))
        row0 = 0 if rng.random() < 0.5 else int(rng.integers(0, length))
        n_rows = length - row0 if rng.random() < 0.5 else int(rng.integers(1, length - row0 + 1))
        chunk = 0 if rng.random() < 0.3 else int(rng.integers(1, n_rows + 1))
        hq, hkv = _HEADS[(3 * i + 1) % len(_HEADS)]
        draws.append(dict(w=dict(mode="prefill", seq_lens=(length,), topk=[1, 50, 256, 1000, 3000][i % 5],
                                 n_layers=int(rng.integers(1, 5)), hq=hq, hkv=hkv, d_idx=int(rng.choice([64, 128])),
                                 needles=int(rng.choice([0, 2])), seed=2000 + i, name=f"random_prefill_{i}"),
                          row0=row0, n_rows=n_rows, chunk=chunk))
    return draws


@pytest.mark.parametrize("draw", _decode_draws(), ids=lambda d: d["name"])
def test_step_decode_random_shapes(draw):
    """A seeded random decode shape: every row against the C++ oracle, both schedules."""
    w = cs.custom(**draw)
    dw = device_workload(w)
    ref = _cpp_rows(w, range(w.n_rows))
    for schedule in (clsa.SCHEDULE_LAYER_BATCHED, clsa.SCHEDULE_PER_LAYER):
        idx, cnt, out = _run_step(dw, schedule)
        dev = bf16_dev_to_f64(out)
        for r in range(w.n_rows):
            assert cnt[r] == ref["count"][r] == min(w.topk, w.row_len(r)), (schedule, r)
            assert np.array_equal(idx[r], ref["idx"][r]), f"schedule {schedule} row {r}: index mismatch"
            assert_outputs_close(dev[r], ref["out"][r], f"{w.name} schedule {schedule} row {r}")
    _say(f"{w.name}: B={w.batch} k={w.topk} L={w.n_layers} hq/hkv={w.hq}/{w.hkv} d_idx={w.d_idx} match")


@pytest.mark.parametrize("draw", _prefill_draws(), ids=lambda d: d["w"]["name"])
def test_step_prefill_random_shapes(draw):
    """A seeded random prefill call (start position, row count and chunk drawn too): every row of
    the call, or about 150 of them for long calls, against the C++ oracle, both schedules."""
    w = cs.custom(**draw["w"])
    dw = device_workload(w)
    row0, n_rows, chunk = draw["row0"], draw["n_rows"], draw["chunk"]
    pos = list(range(row0, row0 + n_rows))
    if len(pos) > 150:
        pos = sorted(set(pos[::len(pos) // 100]) | set(pos[-20:]) | {p for p in pos if abs(p - w.topk) <= 2})
    ref = _cpp_rows(w, pos)
    for schedule in (clsa.SCHEDULE_LAYER_BATCHED, clsa.SCHEDULE_PER_LAYER):
        idx, cnt, out = _run_step(dw, schedule, rows_kw=dict(row0=row0, n_rows=n_rows), chunk=chunk)
        assert np.array_equal(cnt, np.minimum(np.arange(row0 + 1, row0 + n_rows + 1), w.topk))
        dev = bf16_dev_to_f64(out)
        for i, t in enumerate(pos):
            assert np.array_equal(idx[t - row0], ref["idx"][i]), f"schedule {schedule} position {t}: index mismatch"
            assert_outputs_close(dev[t - row0], ref["out"][i], f"{w.name} schedule {schedule} position {t}")
    _say(f"{w.name}: rows {row0}..{row0 + n_rows - 1} chunk {chunk} k={w.topk} L={w.n_layers} "
         f"hq/hkv={w.hq}/{w.hkv}: {len(pos)} positions match")
