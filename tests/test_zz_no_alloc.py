"""clsa_step_no_alloc, the step on the library's static per-GPU scratch (for callers that cannot
allocate device memory), against clsa_step with a caller workspace, through the C ABI: two calls in
a row, the second with a smaller input, so the second runs on the scratch the first left behind.
The same kernels run on both paths and every result is deterministic, so indices, counts and
outputs must match bit for bit; the second call's rows are also checked against the C++ oracle."""
import numpy as np
import pytest
import torch

import clsa_synth as cs
import cross_layer_token_amd as clsa
from _gpu_helpers import assert_outputs_close, bf16_dev_to_f64, device_workload, dims_of, rows_of, workspace

pytestmark = pytest.mark.gpu


def _say(*a):
    print(*a, flush=True)


def _buffers(w, R, routing=False):
    L = w.n_layers
    out = torch.full((R, L, w.hq, 128), 7, dtype=torch.int16, device="cuda")
    shape_i = (L, R, w.topk) if routing else (R, w.topk)
    idx = torch.full(shape_i, -7, dtype=torch.int32, device="cuda")
    cnt = torch.full(shape_i[:-1], -7, dtype=torch.int32, device="cuda")
    return out, idx, cnt


def _both(w, schedule=clsa.SCHEDULE_LAYER_BATCHED, chunk=0):
    """(clsa_step with a workspace, clsa_step_no_alloc) results on the same inputs."""
    dw = device_workload(w)
    dims, rows = dims_of(dw), rows_of(dw)
    R = rows.n_rows
    routing = schedule == clsa.SCHEDULE_PER_LAYER_ROUTING
    q_idx = dw.layer_q_idx() if routing else dw.q_idx
    ws, nws = workspace(dims, rows, schedule, chunk)
    ref = _buffers(w, R, routing)
    clsa.step(dims, rows, q_idx, dw.k_idx, dw.k_cache, dw.v_cache, dw.cu_seqlens, dw.q, *ref, ws, nws,
              schedule=schedule, prefill_chunk_rows=chunk)
    del ws
    got = _buffers(w, R, routing)
    clsa.step_no_alloc(dims, rows, q_idx, dw.k_idx, dw.k_cache, dw.v_cache, dw.cu_seqlens, dw.q, *got,
                       schedule=schedule, prefill_chunk_rows=chunk)
    torch.cuda.synchronize()
    return ref, got


def _same(ref, got, what):
    assert torch.equal(ref[1], got[1]), f"{what}: indices differ"
    assert torch.equal(ref[2], got[2]), f"{what}: counts differ"
    assert torch.equal(ref[0], got[0]), f"{what}: outputs differ"


def test_no_alloc_step_equals_step_two_calls_second_smaller():
    big = cs.custom(seq_lens=(100000, 70000, 90000, 120000), d_idx=128, topk=2048, n_layers=4, hq=16, hkv=4,
                    needles=4, seed=91, name="no_alloc_big")
    small = cs.custom(seq_lens=(3000, 700, 5000), d_idx=64, topk=256, n_layers=2, hq=8, hkv=2, needles=2, seed=92,
                      name="no_alloc_small")
    ref, got = _both(big)
    _same(ref, got, "first call (4 rows of up to 120000 tokens)")
    _say("no-alloc first call: identical to clsa_step")
    ref, got = _both(small)
    _same(ref, got, "second call (3 shorter rows)")
    from oracle import cpp as C
    res = C.oracle_rows(small, range(small.n_rows), threads=4)
    dev = bf16_dev_to_f64(got[0])
    idx = got[1].cpu().numpy()
    for r in range(small.n_rows):
        assert np.array_equal(idx[r], res["idx"][r]), f"row {r}"
        assert_outputs_close(dev[r], res["out"][r], f"no-alloc row {r}")
    _say("no-alloc second call: identical to clsa_step and to the oracle")


@pytest.mark.parametrize("schedule", [clsa.SCHEDULE_PER_LAYER, clsa.SCHEDULE_PER_LAYER_ROUTING])
def test_no_alloc_other_decode_schedules(schedule):
    w = cs.custom(seq_lens=(20000, 9000), d_idx=128, topk=512, n_layers=3, hq=8, hkv=2, needles=2, seed=93,
                  name="no_alloc_sched")
    ref, got = _both(w, schedule)
    _same(ref, got, f"schedule {schedule}")


def test_no_alloc_prefill_chunks():
    w = cs.custom(mode="prefill", seq_lens=(3000,), d_idx=128, topk=512, n_layers=2, hq=8, hkv=2, seed=94,
                  name="no_alloc_prefill")
    ref, got = _both(w, chunk=1024)
    _same(ref, got, "prefill")



def test_no_alloc_step_under_graph_capture():
    """The use the entry point exists for: clsa_step_no_alloc captured into a HIP graph (through
    torch.cuda.graph) and replayed three times, with eager work and synchronisations between the
    replays; every replay equals the eager clsa_step bit for bit.  The step clears its tickets with
    its own kernels, so the graph records no memset."""
    w = cs.custom(seq_lens=(30000, 20000, 26000), d_idx=128, topk=1024, n_layers=3, hq=8, hkv=2, needles=2, seed=95,
                  name="no_alloc_graph")
    ref, got = _both(w)
    _same(ref, got, "eager")
    dw = device_workload(w)
    dims, rows = dims_of(dw), rows_of(dw)
    out, idx, cnt = _buffers(w, rows.n_rows)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):  # warm up on the capture stream (the scratch address is looked up here)
        clsa.step_no_alloc(dims, rows, dw.q_idx, dw.k_idx, dw.k_cache, dw.v_cache, dw.cu_seqlens, dw.q, out, idx, cnt)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        clsa.step_no_alloc(dims, rows, dw.q_idx, dw.k_idx, dw.k_cache, dw.v_cache, dw.cu_seqlens, dw.q, out, idx, cnt)
    for rep in range(3):
        out.fill_(7)
        idx.fill_(-7)
        cnt.fill_(-7)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        _same(ref, (out, idx, cnt), f"graph replay {rep}")
        _ = (dw.q.float() * 0).sum().item()  # eager work between the replays
    _say("no-alloc step: three graph replays identical to the eager step")
