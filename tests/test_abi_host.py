"""The C-ABI library on a machine without a GPU: it loads, exports every declared entry point,
and rejects bad arguments on the host before any launch (no compute call is made here)."""
import ctypes
import os
import re

import pytest

from cross_layer_token_amd import binding as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
FAKE = 0x7F0000000000  # 256-byte aligned stand-in address; never dereferenced by these tests


def _declared_functions():
    text = open(os.path.join(ROOT, "include", "clsa.h")).read()
    return sorted(set(re.findall(r"^\s*(?:const\s+)?[a-z_0-9]+\*?\s+\*?(clsa_[a-z_]+)\(", text, re.M)))


def test_header_declares_the_five_entry_points_and_helpers():
    names = _declared_functions()
    for f in ["clsa_index_scores", "clsa_topk", "clsa_gather_kv", "clsa_sparse_attn", "clsa_step",
              "clsa_workspace_bytes", "clsa_status_string", "clsa_last_error_message", "clsa_abi_version"]:
        assert f in names, f


def test_library_exports_every_declared_symbol():
    lib = ctypes.CDLL(B.LIB_PATH)
    for f in _declared_functions():
        assert hasattr(lib, f), f
    assert set(_declared_functions()) == set(B.FUNCTIONS)
    assert B.LIB.clsa_abi_version() == 1


def test_synth_library_exports():
    lib = ctypes.CDLL(os.path.join(ROOT, "clsa_synth", "libclsa_synth.so"))
    for f in ["synth_fill_uniform_int", "synth_fill_normal", "synth_plant_needles", "synth_tensor_key"]:
        assert hasattr(lib, f)


def test_host_tensor_key_matches_python_generator():
    from clsa_synth import gen
    lib = ctypes.CDLL(os.path.join(ROOT, "clsa_synth", "libclsa_synth.so"))
    lib.synth_tensor_key.argtypes = [ctypes.c_uint64, ctypes.c_uint32]
    lib.synth_tensor_key.restype = ctypes.c_uint64
    for seed, tid in [(0, 1), (3, 5), (2 ** 63 + 11, 7)]:
        assert lib.synth_tensor_key(seed, tid) == int(gen.tensor_key(seed, tid))


def test_status_strings():
    assert B.status_string(0) == "CLSA_OK"
    assert B.status_string(3) == "CLSA_ERR_WORKSPACE"


def _dims(**kw):
    d = dict(batch=2, d_idx=128, topk=64, n_layers=2, hq=8, hkv=2)
    d.update(kw)
    return B.make_dims(**d)


def _rows(**kw):
    r = dict(mode=B.MODE_DECODE, n_rows=2, max_row_len=1000, total_tokens=1500, cu_seqlens_host=[0, 1000, 1500])
    r.update(kw)
    return B.make_rows(**r)


def _scores(dims, rows, **over):
    args = dict(q_idx=FAKE, k_idx=FAKE, cu=FAKE, scores=FAKE, ld=1024)
    args.update(over)
    return B.LIB.clsa_index_scores(ctypes.byref(dims), ctypes.byref(rows), args["q_idx"], args["k_idx"], args["cu"],
                                   args["scores"], args["ld"], None)


@pytest.mark.parametrize("dims_kw,rows_kw,over,status,needle", [
    (dict(head_dim=64), {}, {}, B.ERR_UNSUPPORTED, "head_dim"),
    (dict(d_idx=96), {}, {}, B.ERR_UNSUPPORTED, "d_idx"),
    (dict(hq=6, hkv=4), {}, {}, B.ERR_INVALID_ARGUMENT, "multiple of hkv"),
    (dict(topk=0), {}, {}, B.ERR_INVALID_ARGUMENT, "topk"),
    (dict(topk=70000), {}, {}, B.ERR_UNSUPPORTED, "topk"),
    (dict(n_layers=0), {}, {}, B.ERR_INVALID_ARGUMENT, "n_layers"),
    ({}, dict(n_rows=3), {}, B.ERR_INVALID_ARGUMENT, "n_rows == batch"),
    ({}, dict(mode=7), {}, B.ERR_INVALID_ARGUMENT, "mode"),
    ({}, dict(cu_seqlens_host=[0, 1200, 1500]), {}, B.ERR_INVALID_ARGUMENT, "longer than"),
    ({}, dict(cu_seqlens_host=[0, 900, 800]), {}, B.ERR_INVALID_ARGUMENT, "non-decreasing"),
    ({}, dict(cu_seqlens_host=[0, 500, 1400]), {}, B.ERR_INVALID_ARGUMENT, "total_tokens"),
    ({}, dict(cu_seqlens_host=[1, 500, 1500]), {}, B.ERR_INVALID_ARGUMENT, "cu_seqlens[0]"),
    ({}, dict(cu_seqlens_host=[0, 0, 1500]), {}, B.ERR_INVALID_ARGUMENT, "length 0"),
    ({}, dict(max_row_len=2000), {}, B.ERR_INVALID_ARGUMENT, "exceeds total_tokens"),
    ({}, {}, dict(q_idx=0), B.ERR_INVALID_ARGUMENT, "q_idx is NULL"),
    ({}, {}, dict(k_idx=FAKE + 2), B.ERR_INVALID_ARGUMENT, "aligned"),
    ({}, {}, dict(ld=512), B.ERR_INVALID_ARGUMENT, "ld_scores"),
    ({}, dict(mode=B.MODE_PREFILL, n_rows=100, pos0=0, max_row_len=101, seq=0), {}, B.ERR_INVALID_ARGUMENT, "pos0 + n_rows"),
    ({}, dict(mode=B.MODE_PREFILL, n_rows=100, pos0=1000, max_row_len=1100, seq=0, total_tokens=1500), {},
     B.ERR_INVALID_ARGUMENT, "past the end"),
    ({}, dict(mode=B.MODE_PREFILL, n_rows=10, pos0=0, max_row_len=10, seq=2), {}, B.ERR_INVALID_ARGUMENT, "seq"),
])
def test_index_scores_rejects(dims_kw, rows_kw, over, status, needle):
    s = _scores(_dims(**dims_kw), _rows(**rows_kw), **over)
    assert s == status
    assert needle in B.last_error()


def test_topk_rejects_small_workspace():
    dims, rows = _dims(), _rows(max_row_len=50000, total_tokens=60000, cu_seqlens_host=[0, 50000, 60000])
    need = B.workspace_bytes(dims, rows)
    assert need > 2 * 50000 * 8  # candidate lists of the long-row select
    s = B.LIB.clsa_topk(ctypes.byref(dims), ctypes.byref(rows), FAKE, FAKE, 50048, FAKE, FAKE, FAKE, 1024, None)
    assert s == B.ERR_WORKSPACE and "needed" in B.last_error()
    s = B.LIB.clsa_topk(ctypes.byref(dims), ctypes.byref(rows), FAKE, FAKE, 50048, FAKE, FAKE, None, need, None)
    assert s == B.ERR_WORKSPACE


def test_sparse_attn_rejects():
    dims, rows = _dims(), _rows()
    L = B.LIB

    def call(lc=2, qs=2 * 8 * 128, os_=2 * 8 * 128, ksel=None, vsel=None, kc=FAKE, vc=FAKE, idx=FAKE):
        return L.clsa_sparse_attn(ctypes.byref(dims), ctypes.byref(rows), FAKE, qs, lc, ksel, vsel, kc, vc, FAKE, idx,
                                  FAKE, FAKE, os_, FAKE, 1 << 40, None)
    assert call(lc=3) == B.ERR_UNSUPPORTED
    assert call(lc=0) == B.ERR_UNSUPPORTED
    assert call(qs=100) == B.ERR_INVALID_ARGUMENT
    assert call(ksel=FAKE) == B.ERR_INVALID_ARGUMENT and "v_sel" in B.last_error()
    assert call(kc=None) == B.ERR_INVALID_ARGUMENT and "k_cache" in B.last_error()


def test_step_rejects():
    dims, rows = _dims(), _rows()
    ws = B.workspace_bytes(dims, rows)

    def call(**kw):
        a = dict(q_idx=FAKE, k_idx=FAKE, k_cache=FAKE, v_cache=FAKE, cu_seqlens=FAKE, q=FAKE, out=FAKE, idx=FAKE,
                 count=FAKE, scores=None, ld_scores=0, k_sel=None, v_sel=None, schedule=0, prefill_chunk_rows=0)
        wsz = kw.pop("ws", ws)
        a.update(kw)
        sa = B.StepArgs(**a)
        return B.LIB.clsa_step(ctypes.byref(dims), ctypes.byref(rows), ctypes.byref(sa), FAKE, wsz, None)
    assert call(schedule=5) == B.ERR_INVALID_ARGUMENT
    assert call(out=None) == B.ERR_INVALID_ARGUMENT
    assert call(k_sel=FAKE) == B.ERR_INVALID_ARGUMENT
    assert call(scores=FAKE, ld_scores=10) == B.ERR_INVALID_ARGUMENT
    assert call(ws=ws - 1) == B.ERR_WORKSPACE
    assert call(prefill_chunk_rows=-1) == B.ERR_INVALID_ARGUMENT
    # the per-layer routing ablation: decode only, no caller scores or compact buffers
    wsr = B.workspace_bytes(dims, rows, B.SCHEDULE_PER_LAYER_ROUTING)
    assert wsr > 0
    assert call(schedule=B.SCHEDULE_PER_LAYER_ROUTING, scores=FAKE, ld_scores=4096, ws=wsr) == B.ERR_INVALID_ARGUMENT
    pre = B.make_rows(B.MODE_PREFILL, 100, 100, 4096, seq=0, pos0=0)
    sa = B.StepArgs(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None, 0, None, None,
                    B.SCHEDULE_PER_LAYER_ROUTING, 0)
    st = B.LIB.clsa_step(ctypes.byref(dims), ctypes.byref(pre), ctypes.byref(sa), FAKE, 1 << 30, None)
    assert st == B.ERR_UNSUPPORTED and "DECODE" in B.last_error()


def test_index_project_rejects():
    dims, rows = _dims(), _rows()

    def call(rows_=rows, d_model=4096, h=FAKE, wq=FAKE, wk=FAKE, cu=FAKE, q_idx=FAKE, k_idx=FAKE, k_new=None,
             v_new=None, kc=None, vc=None):
        return B.LIB.clsa_index_project(ctypes.byref(dims), ctypes.byref(rows_), d_model, h, wq, wk, cu, q_idx,
                                        k_idx, k_new, v_new, kc, vc, None)
    pre = B.make_rows(B.MODE_PREFILL, 100, 100, 1500, seq=0, pos0=0)
    assert call(rows_=pre) == B.ERR_UNSUPPORTED and "DECODE" in B.last_error()
    assert call(d_model=48) == B.ERR_UNSUPPORTED and "d_model" in B.last_error()
    assert call(d_model=0) == B.ERR_UNSUPPORTED
    assert call(d_model=65536 + 32) == B.ERR_UNSUPPORTED
    assert call(h=None) == B.ERR_INVALID_ARGUMENT and "h is NULL" in B.last_error()
    assert call(wk=FAKE + 8) == B.ERR_INVALID_ARGUMENT and "aligned" in B.last_error()
    assert call(k_idx=None) == B.ERR_INVALID_ARGUMENT and "k_idx" in B.last_error()
    assert call(k_new=FAKE) == B.ERR_INVALID_ARGUMENT and "together" in B.last_error()
    assert call(k_new=FAKE, v_new=FAKE) == B.ERR_INVALID_ARGUMENT and "k_cache" in B.last_error()
    assert call(rows_=_rows(cu_seqlens_host=[0, 0, 1500])) == B.ERR_INVALID_ARGUMENT


def test_distill_rejects():
    dims = _dims()
    pre = B.make_rows(B.MODE_PREFILL, 100, 100, 1500, seq=0, pos0=0, cu_seqlens_host=[0, 1000, 1500])
    nws = B.distill_workspace_bytes(dims, pre)
    assert nws >= 100 * (2 * 8 + 1 + 1) * 4

    def call(rows_=pre, q=FAKE, qs=2 * 8 * 128, kc=FAKE, sc=FAKE, ld=128, kl=FAKE, loss=None, ws=FAKE, wsz=nws):
        return B.LIB.clsa_distill_kl(ctypes.byref(dims), ctypes.byref(rows_), q, qs, kc, FAKE, sc, ld, kl, loss, ws,
                                     wsz, None)
    assert call(rows_=_rows()) == B.ERR_UNSUPPORTED and "PREFILL" in B.last_error()
    assert B.LIB.clsa_distill_workspace_bytes(ctypes.byref(dims), ctypes.byref(_rows())) == 0
    assert call(q=None) == B.ERR_INVALID_ARGUMENT and "q is NULL" in B.last_error()
    assert call(kc=FAKE + 4) == B.ERR_INVALID_ARGUMENT and "aligned" in B.last_error()
    assert call(qs=100) == B.ERR_INVALID_ARGUMENT
    assert call(ld=64) == B.ERR_INVALID_ARGUMENT and "ld_scores" in B.last_error()
    assert call(loss=FAKE + 2) == B.ERR_INVALID_ARGUMENT and "loss" in B.last_error()
    assert call(wsz=nws - 1) == B.ERR_WORKSPACE
    assert call(ws=None) == B.ERR_WORKSPACE


def test_workspace_sizes_cover_every_call():
    # 128K decode: candidate lists dominate; per-layer schedule adds the two compact buffers
    dims = B.make_dims(16, 128, 2048, 16, 32, 8)
    rows = B.make_rows(B.MODE_DECODE, 16, 131072, 16 * 131072)
    batched = B.workspace_bytes(dims, rows, B.SCHEDULE_LAYER_BATCHED)
    per_layer = B.workspace_bytes(dims, rows, B.SCHEDULE_PER_LAYER)
    assert batched >= 16 * 131072 * 8 + 16 * 131072 * 4
    assert per_layer >= 2 * 16 * 8 * 2048 * 128 * 2 + 16 * 131072 * (8 + 4)
    with pytest.raises(B.CLSAError):
        B.workspace_bytes(B.make_dims(16, 128, 2048, 16, 32, 8, head_dim=64), rows)


def test_attention_split_ranges_stay_inside_the_row(tmp_path):
    """The attention's per-split selection range (split_key_range, shared by host and device code)
    clamps any count a caller passes into [0, k]: compiled with g++ and swept over counts below 0,
    at 0, above k and far above k, every position read stays below k and the splits cover exactly
    the clamped count."""
    import subprocess
    here = os.path.dirname(os.path.abspath(__file__))
    exe = str(tmp_path / "split_bounds")
    subprocess.run(["g++", "-std=c++17", "-O1", "-Wall", "-o", exe, os.path.join(here, "host", "split_bounds.cpp")],
                   check=True)
    r = subprocess.run([exe], stdout=subprocess.PIPE, text=True)
    assert r.returncode == 0 and r.stdout.startswith("ok"), r.stdout


def test_step_no_alloc_rejects_a_step_beyond_its_scratch():
    """clsa_step_no_alloc refuses, on the host and before any HIP call, a step whose workspace
    exceeds its static scratch: 64 rows of 131072 tokens (their scores and candidate lists alone
    pass 64 MiB)."""
    R, n = 64, 131072
    dims = _dims(batch=R, topk=2048)
    rows = B.make_rows(B.MODE_DECODE, R, n, R * n)
    with pytest.raises(B.CLSAError) as e:
        B.step_no_alloc(dims, rows, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, stream=0)
    assert e.value.status == B.ERR_UNSUPPORTED and "static scratch" in str(e.value)
    assert B.NO_ALLOC_SCRATCH_BYTES == 64 << 20
    # a NULL argument is reported before the size
    with pytest.raises(B.CLSAError) as e:
        B.step_no_alloc(dims, rows, None, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, stream=0)
    assert e.value.status == B.ERR_INVALID_ARGUMENT


def test_prefill_score_tiles_cover_the_causal_triangle_once(tmp_path):
    """The prefill score kernel's grid enumerates only the causal 128 x 128 tiles: compiled with g++
    (with the address and undefined-behaviour sanitizers) and swept over call offsets and row
    counts, every tile index maps to a distinct causal tile and every causal tile is reached."""
    import subprocess
    here = os.path.dirname(os.path.abspath(__file__))
    exe = str(tmp_path / "prefill_tiles")
    subprocess.run(["g++", "-std=c++17", "-O1", "-Wall", "-fsanitize=address,undefined", "-o", exe,
                    os.path.join(here, "host", "prefill_tiles.cpp")], check=True)
    r = subprocess.run([exe], stdout=subprocess.PIPE, text=True, env={**os.environ, "LD_PRELOAD": ""})
    assert r.returncode == 0 and r.stdout.startswith("ok"), r.stdout


def test_distill_kl_tiles_cover_the_causal_triangle_once(tmp_path):
    """The distillation KL pass launches one workgroup per causal 32-position x 256-key tile: compiled
    with g++ (with the address and undefined-behaviour sanitizers) and swept over call offsets and
    row counts, every tile index maps to a distinct tile holding a visible (position, key) pair, and
    every such tile is reached; the 2^24-position call, whose tiles fill more than one grid row, maps
    its ends correctly."""
    import subprocess
    here = os.path.dirname(os.path.abspath(__file__))
    exe = str(tmp_path / "distill_tiles")
    subprocess.run(["g++", "-std=c++17", "-O1", "-Wall", "-fsanitize=address,undefined", "-o", exe,
                    os.path.join(here, "host", "distill_tiles.cpp")], check=True)
    r = subprocess.run([exe], stdout=subprocess.PIPE, text=True, env={**os.environ, "LD_PRELOAD": ""})
    assert r.returncode == 0 and r.stdout.startswith("ok"), r.stdout


def test_per_layer_workspace_gathers_in_cache_sized_chunks():
    """The per-layer decode schedule gathers the compact K_S/V_S of a chunk of rows at a time (at most
    192 MiB, inside the 256 MB Infinity Cache): for 64 rows of 131072 tokens with k = 2048 and 8 KV
    heads (8 MiB of K_S/V_S per row) its workspace holds 24 rows of compact buffers, not 64."""
    R, n = 64, 131072
    dims = _dims(batch=R, topk=2048, hq=32, hkv=8, n_layers=12)
    rows = B.make_rows(B.MODE_DECODE, R, n, R * n)
    batched = B.workspace_bytes(dims, rows, B.SCHEDULE_LAYER_BATCHED)
    per_layer = B.workspace_bytes(dims, rows, B.SCHEDULE_PER_LAYER)
    per_row = 2 * 8 * 2048 * 128 * 2
    # the compact buffers of 24 rows, plus the per-layer passes' own split partials
    assert 24 * per_row <= per_layer - batched <= 24 * per_row + (16 << 20)


# ---- workspace sizing over arbitrary arguments -------------------------------------------------
# The sizing calls validate and plan on the host only, so any argument values may be tried here;
# under tests/test_sanitizers.py this runs against the address- and undefined-behaviour-sanitized
# build, where a signed overflow or an out-of-bounds read in the planning aborts the run.
def _sizing_args():
    from hypothesis import strategies as st
    i32 = st.one_of(st.integers(-3, 3), st.sampled_from([31, 32, 33, 63, 64, 127, 128, 255, 256, 257, 2047, 2048,
                                                          2049, 8192, 12288, 12289, 65535, 65536, 65537, 2**20,
                                                          2**24 - 1, 2**24, 2**24 + 1, 2**30, 2**31 - 1, -(2**31)]),
                    st.integers(-(2**31), 2**31 - 1))
    return dict(batch=st.one_of(st.integers(1, 9), i32), d_idx=st.sampled_from([-1, 0, 32, 64, 96, 128, 256]),
                topk=i32, n_layers=st.one_of(st.integers(-1, 20), i32), hq=st.one_of(st.integers(-1, 64), i32),
                hkv=st.one_of(st.integers(-1, 16), i32), head_dim=st.sampled_from([64, 128, 128, 128]),
                sm_scale=st.sampled_from([0.0, -1.0, 0.088, 1.0, float("nan"), float("inf")]),
                mode=st.sampled_from([0, 1, 1, 0, 2, -1]), n_rows=i32, seq=st.one_of(st.integers(-1, 9), i32),
                pos0=i32, max_row_len=i32, total_tokens=st.one_of(i32, st.integers(-(2**63), 2**63 - 1)),
                cu=st.one_of(st.none(), st.lists(st.integers(-5, 2**24 + 5), min_size=1, max_size=10)),
                schedule=st.sampled_from([0, 1, 2, 3, -1]), chunk=st.one_of(st.integers(-2, 3), i32))


def test_workspace_sizing_never_fails_uncleanly():
    """Any clsa_dims / clsa_rows contents, schedule and chunk: the sizing calls return 0 with an
    error message or a positive size that is a multiple of 256, and never crash or overflow."""
    pytest.importorskip("hypothesis")
    from hypothesis import HealthCheck, given, settings

    @settings(max_examples=600, deadline=None, derandomize=True, database=None,
              suppress_health_check=list(HealthCheck))
    @given(**_sizing_args())
    def check(batch, d_idx, topk, n_layers, hq, hkv, head_dim, sm_scale, mode, n_rows, seq, pos0, max_row_len,
              total_tokens, cu, schedule, chunk):
        dims = B.Dims(batch, d_idx, topk, n_layers, hq, hkv, head_dim, sm_scale)
        # a host cu_seqlens must hold batch + 1 entries; a shorter list is only passed for a
        # batch it fits (reading past a caller's array is the caller's contract, not tested here)
        host = cu if cu is not None and 1 <= batch <= len(cu) - 1 else None
        rows = B.make_rows(mode, n_rows, max_row_len, total_tokens, seq=seq, pos0=pos0,
                           cu_seqlens_host=host[:batch + 1] if host is not None else None)
        for n in (B.LIB.clsa_workspace_bytes(ctypes.byref(dims), ctypes.byref(rows), schedule, chunk),
                  B.LIB.clsa_distill_workspace_bytes(ctypes.byref(dims), ctypes.byref(rows))):
            if n == 0:
                assert B.last_error(), "a zero size must leave an error message"
            else:
                assert n % 256 == 0, n

    check()
