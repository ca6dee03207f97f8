"""Throughput of the CLSA decode step on one MI355X.

    python bench.py [--steps K] [--warmup W] [--config 3] [--gpus 1]

One step = routing scores over the whole shared cache + top-k once + all L layers of sparse
attention over the selection (clsa_step, layer-batched), on inputs already resident in HBM.
Prints one JSON line.  ``value`` is decoded tokens/s of the whole step (B tokens per step).
``roofline`` covers the dominant kernel (the routing-score stream over K_idx), timed live with
HIP events on the launch stream; ``cpu_baseline`` times the fp64 oracle on the host.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
HBM_PEAK_GBPS = 8000.0
MFMA_BF16_PEAK_TFLOPS = 2500.0
# v_exp_f32 per second: 256 CUs x 4 SIMDs x 16 lanes at a quarter of the full rate, at 2.4 GHz
EXP2_PEAK_PER_S = 256 * 4 * 16 / 4 * 2.4e9
METRIC = "decode tokens/sec + HBM GB/s (% roofline), index+top-k+L-layer attn at 128K"
# hidden width of the new-token indexer projections timed beside the step (the pages give none;
# a round width of the order of the 4B-parameter models they evaluate)
APPEND_D_MODEL = 4096
INDEX_KERNEL_SOURCES = ["cross_layer_token_amd/csrc/k_index.hip", "cross_layer_token_amd/csrc/select_common.h",
                        "cross_layer_token_amd/csrc/device_common.h", "cross_layer_token_amd/csrc/clsa_internal.h"]
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic_index_scores_decode_b16_n128k.json")


def algorithmic_bytes(w) -> dict:
    """Bytes the method must move per decode step: the K_idx scan once, each selected K and V row
    once, the queries and outputs of every layer, and the index output."""
    kidx = q_idx = kv = qo = idx = 0
    row_kv = 2 * w.hkv * w.head_dim  # one token's K (or V) row, bytes
    for n in w.seq_lens:
        m = min(w.topk, n)
        kidx += 2 * w.d_idx * n
        q_idx += 2 * w.d_idx
        kv += 2 * row_kv * m
        idx += 4 * m
    qo = 2 * 2 * w.batch * w.n_layers * w.hq * w.head_dim
    return {"k_idx": kidx, "q_idx": q_idx, "kv_selected": kv, "q_and_out": qo, "indices": idx,
            "total": kidx + q_idx + kv + qo + idx}


def index_kernel_sha() -> str:
    h = hashlib.sha256()
    for p in INDEX_KERNEL_SOURCES:
        h.update(open(os.path.join(ROOT, p), "rb").read())
    return h.hexdigest()[:16]


def measured_traffic(bytes_alg_launch: float):
    """HBM bytes per launch of the score kernel from the committed rocprofv3 counter summary,
    if it was taken on the current kernel source; otherwise None."""
    try:
        t = json.load(open(TRAFFIC_FILE))
    except (OSError, ValueError):
        return None
    if t.get("kernel_source_sha") != index_kernel_sha():
        return None
    return t.get("traffic_bytes_per_launch")


# ---- rocprofv3 summaries (text under profiles/, made from rocprofv3's own CSV output) ----------
WORKLOAD_TAG = "decode_b16_n128k"
PROFILE_COMMANDS = {
    "trace": "rocprofv3 --kernel-trace --stats --output-format csv -d rocprof_out/trace -o bench -- "
             "python3 bench.py --steps 20 --warmup 3 --no-cpu-baseline --no-prefill --no-decode-configs",
    "fetch": "rocprofv3 --pmc FETCH_SIZE --output-format csv -d rocprof_out/fetch -o bench -- "
             "python3 bench.py --steps 3 --warmup 1 --no-cpu-baseline --no-per-layer --no-prefill --no-append "
             "--no-distill --no-decode-configs --profile-copy-mib 1024",
    "write": "rocprofv3 --pmc WRITE_SIZE --output-format csv -d rocprof_out/write -o bench -- "
             "python3 bench.py --steps 3 --warmup 1 --no-cpu-baseline --no-per-layer --no-prefill --no-append "
             "--no-distill --no-decode-configs --profile-copy-mib 1024",
}


def _csv_rows(path):
    import csv
    with open(path, newline="") as f:
        return list(csv.DictReader(f))


def _short_kernel(name: str) -> str:
    n = name.replace("(anonymous namespace)::", "").split("(")[0]
    for pre in ("void ", "clsa::", "at::native::"):
        n = n.replace(pre, "")
    return n.strip()


def summarize_trace(trace_dir: str) -> str:
    """Markdown table of rocprofv3's kernel statistics (``*_kernel_stats.csv``)."""
    import glob
    path = sorted(glob.glob(os.path.join(trace_dir, "*_kernel_stats.csv")))[0]
    lines = [f"# Kernel trace: decode step, {WORKLOAD_TAG}", "",
             "Made by (on one MI355X):", "", f"    {PROFILE_COMMANDS['trace']}",
             f"    python bench.py --summarize-trace {trace_dir}", "",
             "The run holds warmup + timed steps of the layer-batched step (score kernel with histogram,",
             "top-k select, sparse attention), the score kernel alone (the roofline line), the",
             "per-layer schedule (gather + one attention per layer), the per-layer routing ablation",
             "(scores, top-k and one attention per layer), the new-token indexer projections and cache",
             "append ahead of the step, the Infinity Cache probes (torch reduce and copy) and the",
             "synthetic-input fill.", "",
             "| kernel | calls | avg us | min us | max us | share % |", "|---|---:|---:|---:|---:|---:|"]
    for r in _csv_rows(path):
        lines.append(f"| `{_short_kernel(r['Name'])}` | {r['Calls']} | {float(r['AverageNs']) / 1e3:.2f} | "
                     f"{float(r['MinNs']) / 1e3:.2f} | {float(r['MaxNs']) / 1e3:.2f} | {float(r['Percentage']):.2f} |")
    # The score kernel's launches by kind: the scores-only loop (the roofline line) launches it back
    # to back, while the step and the ablations follow each launch with the top-k select.
    traces = sorted(glob.glob(os.path.join(trace_dir, "*_kernel_trace.csv")))
    if traces:
        tr = sorted(_csv_rows(traces[0]), key=lambda r: int(r["Start_Timestamp"]))
        is_idx = ["k_index_scores_decode" in r["Kernel_Name"] for r in tr]
        alone, other = [], []
        for i, r in enumerate(tr):
            if not is_idx[i]:
                continue
            us = (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3
            back_to_back = (i > 0 and is_idx[i - 1]) or (i + 1 < len(tr) and is_idx[i + 1])
            (alone if back_to_back else other).append(us)
        lines += ["", "`k_index_scores_decode<128>` by kind of launch (from the per-dispatch trace):", "",
                  "| launches | calls | avg us | min us | max us |", "|---|---:|---:|---:|---:|"]
        for name, v in (("scores only, back to back (the roofline line)", alone),
                        ("followed by the top-k select (step, routing ablation, append)", other)):
            if v:
                lines.append(f"| {name} | {len(v)} | {sum(v) / len(v):.2f} | {min(v):.2f} | {max(v):.2f} |")
    return "\n".join(lines) + "\n"


FUSED_ATTN_KERNEL = "k_sparse_attn<true, 2, true, 4, false>"


def summarize_counters(fetch_dir: str, write_dir: str, copy_mib: int = 1024) -> tuple:
    """HBM bytes per launch of the score kernel from FETCH_SIZE / WRITE_SIZE (KiB per dispatch),
    each scaled by what the same counter reads for a plain device copy of copy_mib MiB."""
    import glob
    def rows(d):
        return _csv_rows(sorted(glob.glob(os.path.join(d, "*_counter_collection.csv")))[0])
    out = {}
    for tag, d, cname in (("fetch", fetch_dir, "FETCH_SIZE"), ("write", write_dir, "WRITE_SIZE")):
        rr = [r for r in rows(d) if r["Counter_Name"] == cname]
        copy = max((r for r in rr if "copyBuffer" in r["Kernel_Name"]), key=lambda r: int(r["Grid_Size"]))
        scale = (copy_mib * 1024.0) / float(copy["Counter_Value"])
        # the scores-only launches are the ones after the last attention dispatch (bench order)
        last_attn = max(int(r["Dispatch_Id"]) for r in rr if "k_sparse_attn" in r["Kernel_Name"])
        idx_only = [float(r["Counter_Value"]) for r in rr
                    if "k_index_scores_decode" in r["Kernel_Name"] and int(r["Dispatch_Id"]) > last_attn]
        in_step = [float(r["Counter_Value"]) for r in rr
                   if "k_index_scores_decode" in r["Kernel_Name"] and int(r["Dispatch_Id"]) < last_attn]
        # the step's attention, which also finishes the selection and reads K/V through the index
        attn = [float(r["Counter_Value"]) for r in rr if FUSED_ATTN_KERNEL in r["Kernel_Name"]]
        out[tag] = {"copy_kib": float(copy["Counter_Value"]), "scale": scale,
                    "kib_per_launch": sum(idx_only) / len(idx_only), "launches": len(idx_only),
                    "kib_per_launch_in_step": sum(in_step) / len(in_step),
                    "attn_kib_per_launch": sum(attn) / len(attn) if attn else None, "attn_launches": len(attn)}
    traffic = (out["fetch"]["kib_per_launch"] * out["fetch"]["scale"]
               + out["write"]["kib_per_launch"] * out["write"]["scale"]) * 1024.0
    import clsa_synth as cs
    w = cs.config(3)
    b = algorithmic_bytes(w)
    alg = b["k_idx"] + b["q_idx"] + 4 * w.total_tokens
    rec = {"kernel": "k_index_scores_decode<128>", "workload": WORKLOAD_TAG, "kernel_source_sha": index_kernel_sha(),
           "kernel_sources": INDEX_KERNEL_SOURCES, "traffic_bytes_per_launch": round(traffic),
           "algorithmic_bytes_per_launch": alg, "traffic_over_algorithmic": round(traffic / alg, 4),
           "fetch": out["fetch"], "write": out["write"], "copy_mib": copy_mib,
           "commands": [PROFILE_COMMANDS["fetch"], PROFILE_COMMANDS["write"],
                        f"python bench.py --summarize-counters {fetch_dir} {write_dir}"]}
    md = [f"# HBM traffic of the score kernel, {WORKLOAD_TAG}", "",
          "Made by (on one MI355X; the counter passes run separately):", "",
          *[f"    {c}" for c in rec["commands"]], "",
          f"Calibration: a plain device copy of {copy_mib} MiB reads as FETCH_SIZE "
          f"{out['fetch']['copy_kib']:.2f} KiB and WRITE_SIZE {out['write']['copy_kib']:.2f} KiB, so the factors",
          f"are {out['fetch']['scale']:.4f} (fetch) and {out['write']['scale']:.4f} (write).", "",
          "| | FETCH_SIZE KiB | WRITE_SIZE KiB |", "|---|---:|---:|",
          f"| scores only (per launch, {out['fetch']['launches']} launches) | {out['fetch']['kib_per_launch']:.2f} | "
          f"{out['write']['kib_per_launch']:.2f} |",
          f"| in the step (with the top-k histogram) | {out['fetch']['kib_per_launch_in_step']:.2f} | "
          f"{out['write']['kib_per_launch_in_step']:.2f} |", "",
          f"Scaled traffic per scores-only launch: {traffic:,.0f} B; algorithmic (K_idx + q_idx read, fp32",
          f"scores written): {alg:,} B; ratio {traffic / alg:.4f}.", "",
          f"Kernel source hash (first 16 hex of sha256 over {', '.join(INDEX_KERNEL_SOURCES)}): "
          f"`{rec['kernel_source_sha']}`."]
    if out["fetch"]["attn_kib_per_launch"] is not None and out["write"]["attn_kib_per_launch"] is not None:
        at = (out["fetch"]["attn_kib_per_launch"] * out["fetch"]["scale"]
              + out["write"]["attn_kib_per_launch"] * out["write"]["scale"]) * 1024.0
        at_alg = b["kv_selected"] + b["q_and_out"]
        rec["attn"] = {"kernel": FUSED_ATTN_KERNEL, "traffic_bytes_per_launch": round(at),
                       "algorithmic_bytes_per_launch": at_alg, "traffic_over_algorithmic": round(at / at_alg, 4)}
        md += ["", f"The step's attention, `{FUSED_ATTN_KERNEL}` ({out['fetch']['attn_launches']} launches), from the same runs:", "",
               "| | FETCH_SIZE KiB | WRITE_SIZE KiB |", "|---|---:|---:|",
               f"| per launch | {out['fetch']['attn_kib_per_launch']:.2f} | {out['write']['attn_kib_per_launch']:.2f} |", "",
               f"Scaled traffic per launch: {at:,.0f} B; algorithmic (each selected K and V row read once, the",
               f"queries read and the outputs written): {at_alg:,} B; ratio {at / at_alg:.4f}. The rest is the",
               "selection's candidate lists, the index output and the split partials."]
    return rec, "\n".join(md) + "\n"


def infinity_cache_gbps(stream, mib: int = 128) -> dict:
    """How fast data resident in the 256 MB Infinity Cache can be re-read, measured here: a
    read-only reduction over mib MiB, and a device copy of mib/2 MiB to mib/2 MiB (read+write);
    the faster of the two is taken as the cache rate."""
    import torch
    x = torch.ones(mib << 18, dtype=torch.float32, device="cuda")
    half = x[: x.numel() // 2]
    dst = torch.empty_like(half)

    def rate(fn, nbytes):
        with torch.cuda.stream(stream):
            for _ in range(5):
                fn()
            ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            ev0.record(stream)
            for _ in range(50):
                fn()
            ev1.record(stream)
        torch.cuda.synchronize()
        return nbytes / (ev0.elapsed_time(ev1) / 50 / 1e3) / 1e9

    read = rate(lambda: x.sum(), mib << 20)
    copy = rate(lambda: dst.copy_(half), mib << 20)
    return {"read_gbps": round(read, 1), "copy_gbps": round(copy, 1), "gbps": round(max(read, copy), 1)}


def decode_configs_report(configs=(1, 2, 5), steps: int = 50, warmup: int = 10) -> dict:
    """The layer-batched decode step on the other decode workloads (the single short row, the
    32K batch, and the ragged 64-sequence batch with tie-heavy indexer entries), reported beside
    the 128K line: time per step, tokens/s, and the algorithmic HBM rate against the 8 TB/s peak."""
    import torch

    import clsa_synth as cs
    import cross_layer_token_amd as clsa
    from clsa_synth.device import DeviceWorkload

    out_rep = {}
    stream = torch.cuda.current_stream()
    for ci in configs:
        w = cs.config(ci)
        dw = DeviceWorkload(w)
        dims = clsa.make_dims(**dw.dims())
        rows = clsa.make_rows(**dw.rows())
        R, k = w.n_rows, w.topk
        out = torch.empty((R, w.n_layers, w.hq, 128), dtype=torch.int16, device="cuda")
        idx = torch.empty((R, k), dtype=torch.int32, device="cuda")
        cnt = torch.empty((R,), dtype=torch.int32, device="cuda")
        nws = clsa.workspace_bytes(dims, rows)
        ws = torch.empty(nws, dtype=torch.uint8, device="cuda")

        def run(n):
            for _ in range(n):
                clsa.step(dims, rows, dw.q_idx, dw.k_idx, dw.k_cache, dw.v_cache, dw.cu_seqlens, dw.q, out, idx, cnt,
                          ws, nws, stream=stream)

        run(warmup)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        run(steps)
        torch.cuda.synchronize()
        t = (time.perf_counter() - t0) / steps
        b = algorithmic_bytes(w)["total"]
        out_rep[w.name] = {"rows": R, "tokens": w.total_tokens, "max_row_len": w.max_row_len, "topk": k,
                           "layers": w.n_layers, "ms_per_step": round(t * 1e3, 4), "tokens_per_s": round(R / t, 1),
                           "bytes_alg_per_step": b, "hbm_gbps_alg": round(b / t / 1e9, 1),
                           "roofline_frac": round(b / t / 1e9 / HBM_PEAK_GBPS, 4)}
        del dw, out, idx, cnt, ws
        torch.cuda.empty_cache()
    return out_rep


def prefill_report(steps: int = 3, chunk: int = 8192) -> dict:
    """The causal chunked-prefill step (8192 rows, k=2048, L=8), reported beside the decode line.
    Its attention FLOPs run against the bf16 MFMA peak. Each row gathers its own selection of K/V
    rows (about 60 GB per step, served from the Infinity Cache and L2), so the gather rate is
    reported too. The indexer GEMM is also timed alone."""
    import torch

    import clsa_synth as cs
    import cross_layer_token_amd as clsa
    from clsa_synth.device import DeviceWorkload

    w = cs.config(4)
    dw = DeviceWorkload(w)
    dims = clsa.make_dims(**dw.dims())
    rows = clsa.make_rows(**dw.rows())
    R, k, L = w.n_rows, w.topk, w.n_layers
    out = torch.empty((R, L, w.hq, 128), dtype=torch.int16, device="cuda")
    idx = torch.empty((R, k), dtype=torch.int32, device="cuda")
    cnt = torch.empty((R,), dtype=torch.int32, device="cuda")
    nws = clsa.workspace_bytes(dims, rows, clsa.SCHEDULE_LAYER_BATCHED, chunk)
    ws = torch.empty(nws, dtype=torch.uint8, device="cuda")
    stream = torch.cuda.current_stream()

    def run(n):
        for _ in range(n):
            clsa.step(dims, rows, dw.q_idx, dw.k_idx, dw.k_cache, dw.v_cache, dw.cu_seqlens, dw.q, out, idx, cnt,
                      ws, nws, prefill_chunk_rows=chunk, stream=stream)

    run(1)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    run(steps)
    torch.cuda.synchronize()
    t_step = (time.perf_counter() - t0) / steps
    sel = sum(min(k, t + 1) for t in range(R))                  # selected (row, token) pairs
    attn_flop = 4.0 * sel * L * w.hq * w.head_dim                # QK^T and PV, 2 flop per MAC
    gather_bytes = float(sel) * w.hkv * w.head_dim * 2 * 2       # K and V rows each row reads
    # the indexer GEMM alone: causal Q_idx K_idx^T, 2 * d_idx flop per visible (row, token)
    ld = ((R + 63) // 64) * 64
    scores = torch.empty((R, ld), dtype=torch.float32, device="cuda")
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    clsa.index_scores(dims, rows, dw.q_idx, dw.k_idx, dw.cu_seqlens, scores, ld, stream=stream)
    ev0.record(stream)
    for _ in range(10):
        clsa.index_scores(dims, rows, dw.q_idx, dw.k_idx, dw.cu_seqlens, scores, ld, stream=stream)
    ev1.record(stream)
    torch.cuda.synchronize()
    t_idx = ev0.elapsed_time(ev1) / 10 / 1e3
    idx_flop = 2.0 * w.d_idx * (R * (R + 1) // 2)
    return {"workload": w.name, "rows": R, "topk": k, "layers": L, "chunk_rows": chunk, "steps": steps,
            "ms_per_step": round(t_step * 1e3, 3), "tokens_per_s": round(R / t_step, 1),
            "attn_tflops_alg": round(attn_flop / t_step / 1e12, 1),
            "attn_mfma_frac_of_step": round(attn_flop / t_step / 1e12 / MFMA_BF16_PEAK_TFLOPS, 4),
            "gather_bytes": gather_bytes, "gather_tbps": round(gather_bytes / t_step / 1e12, 2),
            "index_gemm_us": round(t_idx * 1e6, 1), "index_gemm_tflops": round(idx_flop / t_idx / 1e12, 1),
            "index_gemm_mfma_frac": round(idx_flop / t_idx / 1e12 / MFMA_BF16_PEAK_TFLOPS, 4)}


def distill_report(reps: int = 3) -> dict:
    """The multi-layer distillation target and loss (eq. 4-5) over all 8192 positions of the
    prefill workload (L = 8, Hq = 32, Hkv = 8), from the routing scores.  Two passes over every
    causal (position, key) pair for each of the L * Hq (layer, head) pairs: bf16 MFMA work against
    its peak, and one exp2 per score and pass against the transcendental rate."""
    import torch

    import clsa_synth as cs
    import cross_layer_token_amd as clsa
    from clsa_synth.device import DeviceWorkload

    w = cs.config(4)
    dw = DeviceWorkload(w)
    dims = clsa.make_dims(**dw.dims())
    rows = clsa.make_rows(**dw.rows())
    R, L, hq = w.n_rows, w.n_layers, w.hq
    ld = ((R + 63) // 64) * 64
    scores = torch.empty((R, ld), dtype=torch.float32, device="cuda")
    stream = torch.cuda.current_stream()
    clsa.index_scores(dims, rows, dw.q_idx, dw.k_idx, dw.cu_seqlens, scores, ld, stream=stream)
    nws = clsa.distill_workspace_bytes(dims, rows)
    ws = torch.empty(nws, dtype=torch.uint8, device="cuda")
    kl = torch.empty(R, dtype=torch.float32, device="cuda")
    loss = torch.empty(1, dtype=torch.float32, device="cuda")

    def run(n):
        for _ in range(n):
            clsa.distill_kl(dims, rows, dw.q, L * hq * 128, dw.k_cache, dw.cu_seqlens, scores, ld, kl, loss, ws, nws,
                            stream=stream)

    run(1)
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    ev0.record(stream)
    run(reps)
    ev1.record(stream)
    torch.cuda.synchronize()
    t = ev0.elapsed_time(ev1) / reps / 1e3
    pairs = R * (R + 1) // 2                          # causal (position, key) pairs
    flop = 2 * pairs * L * hq * w.head_dim * 2         # two passes of q.k, 2 flop per MAC
    exps = 2 * pairs * L * hq                          # one exp2 per score and pass
    return {"workload": w.name, "rows": R, "layers": L, "heads": hq, "reps": reps, "ms": round(t * 1e3, 3),
            "mfma_tflops": round(flop / t / 1e12, 1), "mfma_frac": round(flop / t / 1e12 / MFMA_BF16_PEAK_TFLOPS, 4),
            "exp_per_s": float(f"{exps / t:.4g}"), "exp_frac": round(exps / t / EXP2_PEAK_PER_S, 4),
            "loss": round(float(loss.cpu()[0]), 6)}


def cpu_baseline(w, budget_s: float) -> dict:
    """The fp64 C++ oracle on the host, on a bounded sample of the workload: whole decode rows,
    each evaluated from scratch (inputs regenerated from the generator definition, scores over
    the row's full context, top-k by full sort, all L layers of attention). About budget_s / 2
    on one core, then about budget_s / 2 with the rows spread over the host's cores (at most 16
    threads; each row stays single-threaded)."""
    from oracle import cpp as C

    threads = max(1, min(16, os.cpu_count() or 1))
    one_rows, one_t = 0, 0.0
    while one_t < budget_s / 2 and one_rows < 4 * w.n_rows:
        _, t = C.oracle_rows_timed(w, [one_rows % w.n_rows], threads=1)
        one_t += t
        one_rows += 1
    all_rows, all_t = 0, 0.0
    while all_t < budget_s / 2:
        _, t = C.oracle_rows_timed(w, list(range(w.n_rows)), threads=threads)
        all_t += t
        all_rows += w.n_rows
    return {"value": round(all_rows / all_t, 2), "unit": "tokens/s", "cores": threads, "kind": "oracle",
            "one_core_tokens_per_s": round(one_rows / one_t, 3),
            "sample": f"{w.name}: {all_rows} decode rows on {threads} threads ({all_t:.1f} s) and {one_rows} rows on "
                      f"one thread ({one_t:.1f} s); each row evaluated from scratch by the fp64 C++ oracle (inputs "
                      f"regenerated, scores over the full {w.max_row_len}-token context, top-k by full sort, "
                      f"{w.n_layers}-layer attention)"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--config", type=int, default=3)
    ap.add_argument("--seed", type=int, default=None)
    ap.add_argument("--cpu-budget", type=float, default=20.0, help="seconds of wall time for the oracle baseline")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-per-layer", action="store_true")
    ap.add_argument("--no-prefill", action="store_true", help="skip the prefill report")
    ap.add_argument("--no-append", action="store_true", help="skip the new-token projection + append report")
    ap.add_argument("--no-distill", action="store_true", help="skip the distillation target and loss report")
    ap.add_argument("--no-decode-configs", action="store_true", help="skip the other decode workloads' report")
    ap.add_argument("--profile-copy-mib", type=int, default=0,
                    help="also run one plain device copy of this many MiB (a counter calibration reference)")
    ap.add_argument("--summarize-trace", metavar="DIR", help="write the kernel-trace summary under profiles/ and exit")
    ap.add_argument("--summarize-counters", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"),
                    help="write the score kernel's HBM traffic summary under profiles/ and exit")
    args = ap.parse_args()
    if args.summarize_trace or args.summarize_counters:
        os.makedirs(os.path.join(ROOT, "profiles"), exist_ok=True)
        if args.summarize_trace:
            p = os.path.join(ROOT, "profiles", f"kernel_trace_{WORKLOAD_TAG}.md")
            open(p, "w").write(summarize_trace(args.summarize_trace))
            print("wrote", p)
        if args.summarize_counters:
            rec, md = summarize_counters(*args.summarize_counters)
            json.dump(rec, open(TRAFFIC_FILE, "w"), indent=1)
            p = os.path.join(ROOT, "profiles", f"hbm_traffic_index_scores_{WORKLOAD_TAG}.md")
            open(p, "w").write(md)
            print("wrote", TRAFFIC_FILE, "and", p)
        return
    if args.gpus != 1:
        print("bench.py runs on one GPU only: this build has no multi-GPU path (use --gpus 1)", file=sys.stderr)
        sys.exit(2)

    import torch

    import clsa_synth as cs
    import cross_layer_token_amd as clsa
    from clsa_synth.device import DeviceWorkload

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    w = cs.config(args.config, args.seed)
    if w.mode != "decode":
        print("bench.py times the decode step; the prefill workload is covered by the tests", file=sys.stderr)
        sys.exit(2)
    dw = DeviceWorkload(w)
    dims = clsa.make_dims(**dw.dims())
    rows = clsa.make_rows(**dw.rows())
    R, k = w.n_rows, w.topk
    out = torch.empty((R, w.n_layers, w.hq, 128), dtype=torch.int16, device="cuda")
    idx = torch.empty((R, k), dtype=torch.int32, device="cuda")
    cnt = torch.empty((R,), dtype=torch.int32, device="cuda")
    stream = torch.cuda.current_stream()

    def run_steps(n, schedule, ws, nws):
        for _ in range(n):
            clsa.step(dims, rows, dw.q_idx, dw.k_idx, dw.k_cache, dw.v_cache, dw.cu_seqlens, dw.q, out, idx, cnt, ws,
                      nws, schedule=schedule, stream=stream)

    def timed(fn, n):
        ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        ev0.record(stream)
        fn(n)
        ev1.record(stream)
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
        return ev0.elapsed_time(ev1) / 1e3, wall

    # ---- the step (layer-batched schedule) ------------------------------------------------------
    nws = clsa.workspace_bytes(dims, rows, clsa.SCHEDULE_LAYER_BATCHED)
    ws = torch.empty(nws, dtype=torch.uint8, device="cuda")
    run_steps(args.warmup, clsa.SCHEDULE_LAYER_BATCHED, ws, nws)
    t_gpu, t_wall = timed(lambda n: run_steps(n, clsa.SCHEDULE_LAYER_BATCHED, ws, nws), args.steps)
    t_step = t_wall / args.steps
    balg = algorithmic_bytes(w)
    hbm_gbps = balg["total"] / t_step / 1e9

    # ---- the dominant kernel alone: routing scores streamed from K_idx --------------------------
    ld = ((w.max_row_len + 63) // 64) * 64
    scores = torch.empty((R, ld), dtype=torch.float32, device="cuda")

    def run_scores(n):
        for _ in range(n):
            clsa.index_scores(dims, rows, dw.q_idx, dw.k_idx, dw.cu_seqlens, scores, ld, stream=stream)

    run_scores(args.warmup)
    t_idx, _ = timed(run_scores, args.steps)
    t_idx /= args.steps
    idx_bytes = balg["k_idx"] + balg["q_idx"] + 4 * w.total_tokens   # K_idx + q_idx read, scores written
    achieved = idx_bytes / t_idx / 1e9
    roofline = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                "frac": round(achieved / HBM_PEAK_GBPS, 4), "traffic": measured_traffic(idx_bytes),
                "kernel": "k_index_scores_decode<128>", "bytes_per_launch": idx_bytes,
                "us_per_launch": round(t_idx * 1e6, 2)}

    # ---- dependent-layer schedule (one attention pass per layer), reported beside -----------------
    per_layer = None
    if not args.no_per_layer:
        nws2 = clsa.workspace_bytes(dims, rows, clsa.SCHEDULE_PER_LAYER)
        ws2 = torch.empty(nws2, dtype=torch.uint8, device="cuda")
        run_steps(args.warmup, clsa.SCHEDULE_PER_LAYER, ws2, nws2)
        t2, w2 = timed(lambda n: run_steps(n, clsa.SCHEDULE_PER_LAYER, ws2, nws2), args.steps)
        t_pl = w2 / args.steps
        # its roofline: the step's algorithmic bytes from HBM, plus the compact K_S/V_S read once
        # per layer from the Infinity Cache, at the rate a cache-resident device copy reaches here
        ic = infinity_cache_gbps(stream)
        sel_bytes = 2 * R * w.hkv * w.topk * w.head_dim * 2
        bound = balg["total"] / (HBM_PEAK_GBPS * 1e9) + w.n_layers * sel_bytes / (ic["gbps"] * 1e9)
        per_layer = {"ms_per_step": round(t_pl * 1e3, 4), "tokens_per_s": round(R * args.steps / w2, 1),
                     "hbm_gbps_alg": round(balg["total"] / t_pl / 1e9, 1),
                     "roofline": {"infinity_cache": ic, "compact_bytes_per_layer": sel_bytes,
                                  "bound_ms": round(bound * 1e3, 4), "frac": round(bound / t_pl, 4)}}
        del ws2

    # ---- the ablation without the shared index: route (score + top-k) once per layer ---------------
    routing = None
    if not args.no_per_layer:
        lq = dw.layer_q_idx()
        nws3 = clsa.workspace_bytes(dims, rows, clsa.SCHEDULE_PER_LAYER_ROUTING)
        ws3 = torch.empty(nws3, dtype=torch.uint8, device="cuda")
        idx3 = torch.empty((w.n_layers, R, k), dtype=torch.int32, device="cuda")
        cnt3 = torch.empty((w.n_layers, R), dtype=torch.int32, device="cuda")

        def run_routing(n):
            for _ in range(n):
                clsa.step(dims, rows, lq, dw.k_idx, dw.k_cache, dw.v_cache, dw.cu_seqlens, dw.q, out, idx3, cnt3, ws3,
                          nws3, schedule=clsa.SCHEDULE_PER_LAYER_ROUTING, stream=stream)

        n3 = max(1, args.steps // 5)
        run_routing(max(1, args.warmup // 5))
        _, w3 = timed(run_routing, n3)
        t3 = w3 / n3
        routing = {"ms_per_step": round(t3 * 1e3, 4), "tokens_per_s": round(R / t3, 1), "steps": n3,
                   "vs_shared_routing": round(t3 / t_step, 2)}
        del ws3, idx3, cnt3

    # ---- the step before the routing: new-token indexer projections + cache append ----------------
    append = None
    if not args.no_append:
        d_model = APPEND_D_MODEL
        pin = dw.projection_inputs(d_model)
        q_new = torch.empty((R, w.d_idx), dtype=torch.int16, device="cuda")

        def run_append_steps(n):
            for _ in range(n):
                clsa.index_project(dims, rows, d_model, pin["h"], pin["w_q_idx"], pin["w_k_idx"], dw.cu_seqlens,
                                   q_new, dw.k_idx, pin["k_new"], pin["v_new"], dw.k_cache, dw.v_cache, stream=stream)
                clsa.step(dims, rows, q_new, dw.k_idx, dw.k_cache, dw.v_cache, dw.cu_seqlens, dw.q, out, idx, cnt, ws,
                          nws, stream=stream)

        # weights (query and key projections), hidden states, q_idx and appended rows
        p_bytes = (2 * w.d_idx * d_model + R * d_model + 2 * R * w.d_idx + 2 * R * w.hkv * w.head_dim) * 2
        run_append_steps(args.warmup)
        _, w4 = timed(run_append_steps, args.steps)
        t4 = w4 / args.steps
        # the projection's cost is what it adds to the (device-bound) step; timing the kernel alone
        # from back-to-back host calls would measure the host's call rate instead
        added = t4 - t_step
        append = {"d_model": d_model, "ms_per_step": round(t4 * 1e3, 4), "tokens_per_s": round(R / t4, 1),
                  "added_us_per_step": round(added * 1e6, 2), "project_bytes": p_bytes, "vs_step": round(t4 / t_step, 4)}
        del pin, q_new

    if args.profile_copy_mib > 0:
        n = args.profile_copy_mib << 20
        src = torch.ones(n, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    del dw, out, idx, cnt, ws, scores
    torch.cuda.empty_cache()
    decode_configs = None if args.no_decode_configs else decode_configs_report()
    prefill = None if args.no_prefill else prefill_report()
    distill = None if args.no_distill else distill_report()
    cpu = None if args.no_cpu_baseline else cpu_baseline(w, args.cpu_budget)
    line = {
        "metric": METRIC,
        "value": round(R * args.steps / t_wall, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(t_step * 1e3, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": w.name, "batch": w.batch, "context": w.max_row_len, "d_idx": w.d_idx,
                   "topk": w.topk, "layers": w.n_layers, "hq": w.hq, "hkv": w.hkv, "head_dim": w.head_dim,
                   "schedule": "layer_batched", "seed": w.seed},
        "hbm_gbps": round(hbm_gbps, 1),
        "step_roofline_frac": round(hbm_gbps / HBM_PEAK_GBPS, 4),
        "bytes_alg_per_step": balg["total"],
        "gpu_event_ms_per_step": round(t_gpu / args.steps * 1e3, 4),
        "roofline": roofline,
        "per_layer_schedule": per_layer,
        "per_layer_routing": routing,
        "new_token_append": append,
        "decode_configs": decode_configs,
        "prefill": prefill,
        "distill": distill,
        "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
