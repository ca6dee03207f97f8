"""Parity of clsa_distill_kl (the multi-layer distillation target and loss of eq. 4-5, picx.dev
summary, Methodology, Multi-Layer Distillation) with the fp64 oracle.

Tolerance: the device sums fp32 exponentials and logarithms of fp32 scores, so each KL_t is
compared against the size of the terms it sums, S_t = sum_j A_j (|ln A_j| + |ln softmax(I)_j|):
|KL_dev - KL_ref| <= 2e-6 * S_t + 1e-6.  fp32 rounding is 6e-8 per operation and the hardware
exp2 / log2 are within a few units of it; each lane adds a few hundred terms in sequence before
the fixed-order tree, which grows the relative error of a sum to ~1e-6 at most.  Measured: at
most 2e-7 * S_t on the 8192-position workload.
"""
import numpy as np
import pytest
import torch

import clsa_synth as cs
import cross_layer_token_amd as clsa
from _gpu_helpers import device_workload, dims_of
from clsa_synth import gen
from clsa_synth.device import fill_normal, fill_uniform_int
from oracle import clsa_oracle as O
from oracle.workload_oracle import oracle_distill_row

pytestmark = pytest.mark.gpu

RTOL_TERMS = 2e-6
ATOL = 1e-6


def _say(*a):
    print(*a, flush=True)


def _term_scale(abar, scores):
    s = np.asarray(scores, dtype=np.float64)
    s = s - s.max()
    log_q = s - np.log(np.exp(s).sum())
    a = np.asarray(abar)
    nz = a > 0
    return float(np.sum(a[nz] * (np.abs(np.log(a[nz])) + np.abs(log_q[nz]))))


def _check(dev_kl, ref, what):
    err = abs(float(dev_kl) - ref["kl"])
    bound = RTOL_TERMS * _term_scale(ref["abar"], ref["scores"]) + ATOL
    assert err <= bound, f"{what}: |{dev_kl} - {ref['kl']}| = {err:.3e} > {bound:.3e}"
    return err, bound


def _run(dw, rows_kw=None, q=None, q_idx=None, sm_scale=0.0):
    """Prefill rows of dw: routing scores by clsa_index_scores, then clsa_distill_kl."""
    w = dw.w
    dims = dims_of(dw, sm_scale=sm_scale)
    rows = clsa.make_rows(**dw.rows(**(rows_kw or {})))
    n, r0 = rows.n_rows, (rows_kw or {}).get("row0", 0)
    ld = ((rows.max_row_len + 63) // 64) * 64
    scores = torch.full((n, ld), float("nan"), dtype=torch.float32, device="cuda")
    clsa.index_scores(dims, rows, dw.q_idx[r0:] if q_idx is None else q_idx, dw.k_idx, dw.cu_seqlens, scores, ld)
    nws = clsa.distill_workspace_bytes(dims, rows)
    ws = torch.full((nws,), 0xAB, dtype=torch.uint8, device="cuda")   # content on entry must not matter
    kl = torch.full((n,), float("nan"), dtype=torch.float32, device="cuda")
    loss = torch.full((1,), float("nan"), dtype=torch.float32, device="cuda")
    qq = dw.q[r0:] if q is None else q
    clsa.distill_kl(dims, rows, qq, w.n_layers * w.hq * 128, dw.k_cache, dw.cu_seqlens, scores, ld, kl, loss, ws, nws)
    torch.cuda.synchronize()
    return kl.cpu().numpy().astype(np.float64), float(loss.cpu()[0])


@pytest.mark.parametrize("hq,hkv,L", [(8, 2, 2), (2, 2, 1), (32, 8, 3)])
def test_distill_small_prefill_every_row(hq, hkv, L):
    """600 positions (several 16-, 64- and 512-blocks, ragged ends); (layer, head) pairs per KV
    head from 1 to 12 (one to three waves of the stats workgroup)."""
    w = cs.custom(mode="prefill", seq_lens=(600,), d_idx=64, topk=32, n_layers=L, hq=hq, hkv=hkv, seed=9,
                  name=f"distill_{hq}_{hkv}_{L}")
    dw = device_workload(w)
    kl, loss = _run(dw, rows_kw=dict(row0=0, n_rows=600))
    worst = 0.0
    for r in range(600):
        ref = oracle_distill_row(w, r)
        err, bound = _check(kl[r], ref, f"row {r}")
        worst = max(worst, err / bound)
    assert kl[0] == 0.0 or abs(kl[0]) < 1e-6
    assert abs(loss - kl.mean()) <= 1e-6 * max(1.0, abs(kl.mean()))
    _say(f"hq={hq} hkv={hkv} L={L}: worst error / bound {worst:.3f}, loss {loss:.6f}")


def test_distill_unscaled_form_every_row():
    """sm_scale = 1: the layers' distributions of the raw products q . k, the unscaled form eq. 4
    prints, every row of a 600-position workload against the oracle with scale 1."""
    w = cs.custom(mode="prefill", seq_lens=(600,), d_idx=64, topk=32, n_layers=2, hq=8, hkv=2, seed=9,
                  name="distill_8_2_2")
    dw = device_workload(w)
    kl, loss = _run(dw, rows_kw=dict(row0=0, n_rows=600), sm_scale=1.0)
    worst = 0.0
    for r in range(600):
        ref = oracle_distill_row(w, r, scale=1.0)
        err, bound = _check(kl[r], ref, f"unscaled row {r}")
        worst = max(worst, err / bound)
    assert abs(loss - kl.mean()) <= 1e-6 * max(1.0, abs(kl.mean()))
    _say(f"unscaled: worst error / bound {worst:.3f}, loss {loss:.6f}")


def test_distill_chunk_of_a_later_sequence():
    """Rows 50..549 of the second sequence of a two-sequence cache (pos0 > 0, cache offset)."""
    w = cs.custom(seq_lens=(700, 640), d_idx=128, topk=32, n_layers=2, hq=8, hkv=2, seed=31, name="distill_seq1")
    dw = device_workload(w)
    pos0, n = 50, 500
    L, hq = w.n_layers, w.hq
    q = torch.empty((n, L, hq, 128), dtype=torch.int16, device="cuda")
    q_idx = torch.empty((n, w.d_idx), dtype=torch.int16, device="cuda")
    fill_normal(q, 77, 201)
    fill_uniform_int(q_idx, 77, 202, w.idx_lo, w.idx_hi, w.idx_den)
    torch.cuda.synchronize()
    dims = dims_of(dw)
    cu = w.cu_seqlens
    rows = clsa.make_rows(mode=clsa.MODE_PREFILL, n_rows=n, max_row_len=pos0 + n, total_tokens=w.total_tokens,
                          seq=1, pos0=pos0, cu_seqlens_host=cu.tolist())
    ld = ((pos0 + n + 63) // 64) * 64
    scores = torch.empty((n, ld), dtype=torch.float32, device="cuda")
    clsa.index_scores(dims, rows, q_idx, dw.k_idx, dw.cu_seqlens, scores, ld)
    nws = clsa.distill_workspace_bytes(dims, rows)
    ws = torch.empty(nws, dtype=torch.uint8, device="cuda")
    kl = torch.empty(n, dtype=torch.float32, device="cuda")
    clsa.distill_kl(dims, rows, q, L * hq * 128, dw.k_cache, dw.cu_seqlens, scores, ld, kl, None, ws, nws)
    torch.cuda.synchronize()
    kl = kl.cpu().numpy()
    qh = gen.bf16_bits_to_f64(gen.normal_bf16(77, 201, np.arange(n * L * hq * 128))).reshape(n, L, hq, 128)
    qi = gen.bf16_bits_to_f64(gen.uniform_int_bf16(77, 202, np.arange(n * w.d_idx), w.idx_lo, w.idx_hi,
                                                   w.idx_den)).reshape(n, w.d_idx)
    base = int(cu[1])
    for i in (0, 1, 13, 14, 77, 461, 462, 499):
        t = pos0 + i
        toks = base + np.arange(t + 1)
        abar = O.distill_target(qh[i], gen.bf16_bits_to_f64(w.kv_bits(toks, "k")))
        sc = O.index_scores(qi[i], w.k_idx_f64(toks))
        _check(kl[i], {"abar": abar, "scores": sc, "kl": O.distill_kl(abar, sc)}, f"seq 1 row {i}")


def test_distill_single_row_is_zero_and_calls_are_deterministic():
    w = cs.custom(mode="prefill", seq_lens=(600,), d_idx=64, topk=32, n_layers=2, hq=8, hkv=2, seed=9,
                  name="distill_8_2_2")
    dw = device_workload(w)
    kl1, loss1 = _run(dw, rows_kw=dict(row0=0, n_rows=1))
    assert kl1[0] == 0.0 and loss1 == 0.0
    a, la = _run(dw, rows_kw=dict(row0=0, n_rows=600))
    b, lb = _run(dw, rows_kw=dict(row0=0, n_rows=600))
    assert np.array_equal(a, b) and la == lb


def test_distill_prefill_8k_sampled_rows():
    """The 8192-position prefill workload (L = 8, Hq = 32, Hkv = 8) in one call; rows across the
    16-, 64- and 512-blocks and the needle row checked against the oracle."""
    w = cs.config(4)
    dw = device_workload(w)
    kl, loss = _run(dw)
    assert np.all(np.isfinite(kl)) and np.all(kl >= -1e-4)
    worst = 0.0
    for r in (0, 1, 15, 16, 63, 64, 511, 512, 513, 2047, 4095, 6000, 8191):
        ref = oracle_distill_row(w, r)
        err, bound = _check(kl[r], ref, f"8k row {r}")
        worst = max(worst, err / bound)
        _say(f"8k row {r}: dev {kl[r]:.6f} ref {ref['kl']:.6f} err {err:.2e} bound {bound:.2e}")
    assert abs(loss - kl.mean()) <= 1e-5 * max(1.0, abs(kl.mean()))
    _say(f"8k: worst error / bound {worst:.3f}, loss {loss:.5f}")


def _distill_draws(n=6, seed=5150):
    """Prefill calls drawn from a fixed seed: sequence length, start position and row count, 1 to
    6 layers, one to six query heads per KV head (up to 36 (layer, head) pairs per KV head, past
    one stats workgroup's 32), both indexer widths and three attention scales."""
    heads = [(8, 2), (6, 1), (32, 8), (12, 3), (4, 4), (2, 1)]
    scales = [0.0, 1.0, 0.05]
    rng = np.random.default_rng(seed)
    draws = []
    for i in range(n):
        length = int(rng.integers(40, 901))
        row0 = 0 if i % 2 == 0 else int(rng.integers(1, length))
        n_rows = int(rng.integers(1, length - row0 + 1))
        hq, hkv = heads[i % len(heads)]
        n_layers = 6 if hq // hkv == 6 else int(rng.integers(1, 7))
        draws.append(dict(w=dict(mode="prefill", seq_lens=(length,), d_idx=int(rng.choice([64, 128])), topk=16,
                                 n_layers=n_layers, hq=hq, hkv=hkv, seed=3000 + i,
                                 name=f"distill_random_{i}"),
                          row0=row0, n_rows=n_rows, scale=scales[i % len(scales)]))
    return draws


@pytest.mark.parametrize("draw", _distill_draws(), ids=lambda d: d["w"]["name"])
def test_distill_random_shapes(draw):
    """A seeded random prefill call: up to about 60 of its rows (the first, the last, the rows
    around the 32-position and 256-key block edges and an even spread) against the oracle, and the
    loss against the mean of the call's KL values."""
    w = cs.custom(**draw["w"])
    dw = device_workload(w)
    row0, n_rows, scale = draw["row0"], draw["n_rows"], draw["scale"]
    kl, loss = _run(dw, rows_kw=dict(row0=row0, n_rows=n_rows), sm_scale=scale)
    pos = set(range(row0, row0 + n_rows, max(1, n_rows // 40))) | {row0, row0 + n_rows - 1}
    pos |= {t for t in range(row0, row0 + n_rows) if t % 32 in (0, 31) and t % 256 < 64}
    pos = sorted(pos)[:60] + [row0 + n_rows - 1]
    worst = 0.0
    for t in sorted(set(pos)):
        ref = oracle_distill_row(w, t, scale=None if scale == 0.0 else scale)
        err, bound = _check(kl[t - row0], ref, f"{w.name} position {t}")
        worst = max(worst, err / bound)
    assert abs(loss - kl.mean()) <= 1e-6 * max(1.0, abs(kl.mean()))
    _say(f"{w.name}: positions {row0}..{row0 + n_rows - 1} L={w.n_layers} hq/hkv={w.hq}/{w.hkv} "
         f"scale={scale}: worst error / bound {worst:.3f}")
