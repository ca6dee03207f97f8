"""Throughput of the CLSA decode step on one MI355X.

    python bench.py [--steps K] [--warmup W] [--config 3] [--gpus 1]

One step = routing scores over the whole shared cache + top-k once + all L layers of sparse
attention over the selection (clsa_step, layer-batched), on inputs already resident in HBM.
Prints one JSON line.  ``value`` is decoded tokens/s of the whole step (B tokens per step), from
the median device time of the steps: HIP events around each step, with a 512 MiB read before
every step (outside its events) so that the caches hold nothing of the previous step.
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


def log(*a):
    """A progress line on stderr (the JSON line alone goes to stdout)."""
    print("bench:", *a, file=sys.stderr, flush=True)


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


FLUSH_MIB = 512


class Flush:
    """Evicts the caches between timed calls: a read of FLUSH_MIB MiB (twice the 256 MB Infinity
    Cache) on the timing stream, enqueued before a call and outside its events.  A read evicts as
    well as a write does, and leaves no dirty lines whose write-back the next call would pay for."""

    def __init__(self, stream, mib: int = FLUSH_MIB):
        import torch
        self.stream = stream
        self.mib = mib
        self.buf = torch.ones(mib << 18, dtype=torch.float32, device="cuda")
        self.out = torch.empty((), dtype=torch.float32, device="cuda")

    def __call__(self):
        import torch
        with torch.cuda.stream(self.stream):
            torch.sum(self.buf, dim=0, out=self.out)


def event_times(stream, fn, n: int, flush=None) -> tuple:
    """Device time of each of n calls of fn() on `stream`, from a pair of HIP events around each
    call (flush(), when given, is enqueued before each call, outside its events), and the host wall
    time of the whole loop between two device synchronisations.  Returns (seconds[n], wall)."""
    import torch
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(n)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for a, b in ev:
        if flush is not None:
            flush()
        a.record(stream)
        fn()
        b.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    return np.array([a.elapsed_time(b) / 1e3 for a, b in ev]), wall


def distribution(ts) -> dict:
    """Median, 10th and 90th percentile and mean of per-call times, in ms."""
    t = np.asarray(ts) * 1e3
    return {"median_ms": round(float(np.median(t)), 4), "p10_ms": round(float(np.percentile(t, 10)), 4),
            "p90_ms": round(float(np.percentile(t, 90)), 4), "mean_ms": round(float(t.mean()), 4), "n": int(t.size)}


def cache_flush_check(stream, flush) -> dict:
    """Evidence that the flush evicts: the read rate of a 128 MiB buffer read twice in a row (the
    second read can be served by the Infinity Cache) against the same read right after a flush."""
    import torch
    x = torch.ones(128 << 18, dtype=torch.float32, device="cuda")
    out = torch.empty((), dtype=torch.float32, device="cuda")

    def read():
        with torch.cuda.stream(stream):
            torch.sum(x, dim=0, out=out)

    hot, _ = event_times(stream, read, 20, flush=read)
    cold, _ = event_times(stream, read, 20, flush=flush)
    nbytes = 128 << 20
    return {"read_mib": 128, "hot_gbps": round(nbytes / float(np.median(hot)) / 1e9, 1),
            "after_flush_gbps": round(nbytes / float(np.median(cold)) / 1e9, 1)}


def host_cpu() -> dict:
    """The host's logical CPU count and CPU model name."""
    model = "unknown"
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                model = line.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    return {"nproc": os.cpu_count(), "cpu_model": model}


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
_DECODE_ONLY = "--no-cpu-baseline --no-prefill --no-decode-configs --no-distill"
PROFILE_COMMANDS = {
    "fetch": "rocprofv3 --pmc FETCH_SIZE --output-format csv -d rocprof_out/fetch -o bench -- "
             "python3 bench.py --steps 3 --warmup 1 --no-cpu-baseline --no-per-layer --no-prefill --no-append "
             "--no-distill --no-decode-configs --profile-copy-mib 1024",
    "write": "rocprofv3 --pmc WRITE_SIZE --output-format csv -d rocprof_out/write -o bench -- "
             "python3 bench.py --steps 3 --warmup 1 --no-cpu-baseline --no-per-layer --no-prefill --no-append "
             "--no-distill --no-decode-configs --profile-copy-mib 1024",
}


PREFILL_COUNTER_RUN = "python3 bench.py --prefill-only --prefill-steps 1 --no-distill --profile-copy-mib 1024"
PREFILL_COUNTER_COMMANDS = {
    "mfma": "rocprofv3 --pmc MfmaUtil MfmaFlopsBF16 LdsUtil LdsBankConflict --output-format csv "
            f"-d rocprof_out/prefill_mfma -o bench -- {PREFILL_COUNTER_RUN}",
    "fetch": f"rocprofv3 --pmc FETCH_SIZE --output-format csv -d rocprof_out/prefill_fetch -o bench -- {PREFILL_COUNTER_RUN}",
    "write": f"rocprofv3 --pmc WRITE_SIZE --output-format csv -d rocprof_out/prefill_write -o bench -- {PREFILL_COUNTER_RUN}",
}
PREFILL_KERNELS = (("k_index_scores_prefill<128>", "k_index_scores_prefill"),
                   ("k_prefill_attn (prefill attention)", "k_prefill_attn"),
                   ("k_topk_rows_lds", "k_topk_rows_lds"))
# one pass of eight SQ counters and the GPU's active cycles over the prefill step and the
# distillation passes (their issue and residency picture)
SQ_COUNTERS = ("SQ_WAVE_CYCLES SQ_BUSY_CYCLES SQ_WAIT_ANY SQ_WAIT_INST_ANY SQ_ACTIVE_INST_VALU "
               "SQ_VALU_MFMA_BUSY_CYCLES SQ_ACTIVE_INST_LDS SQ_INSTS_VALU_TRANS_F32 GRBM_GUI_ACTIVE")
SQ_COUNTER_COMMAND = (f"rocprofv3 --pmc {SQ_COUNTERS} --output-format csv -d rocprof_out/prefill_sq -o bench -- "
                      "python3 bench.py --prefill-only --prefill-steps 1")
SQ_KERNELS = (("k_prefill_attn<true>", "k_prefill_attn"), ("k_index_scores_prefill<128>", "k_index_scores_prefill"),
              ("k_topk_rows_lds", "k_topk_rows_lds"), ("k_row_lse", "k_row_lse"),
              ("k_distill_stats", "k_distill_stats"), ("k_distill_kl", "k_distill_kl"))
MI355X_XCDS, MI355X_SIMDS = 8, 1024


def summarize_sq_counters(sq_dir: str) -> str:
    """Issue and residency counters of the prefill and distillation kernels, per launch, from one
    rocprofv3 pass: resident waves per SIMD, the vector-ALU and MFMA busy shares of the SIMDs'
    cycles (rocprofv3's VALUBusy and MfmaUtil), the share of resident wave-cycles spent waiting,
    and the transcendental instructions issued (one v_exp_f32 per score in the distillation)."""
    import glob

    rr = _csv_rows(sorted(glob.glob(os.path.join(sq_dir, "*_counter_collection.csv")))[0])
    by = {}
    for r in rr:
        d = by.setdefault((r["Kernel_Name"], r["Dispatch_Id"]), {"_us": (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3})
        d[r["Counter_Name"]] = d.get(r["Counter_Name"], 0.0) + float(r["Counter_Value"])
    md = ["# Issue and residency counters of the prefill and distillation kernels, prefill_n8k", "",
          "Made by (on one MI355X):", "", f"    {SQ_COUNTER_COMMAND}",
          f"    python bench.py --summarize-sq-counters {sq_dir}", "",
          "The run holds warm-up and timed causal prefill steps of the 8192-row workload (8192 rows in one chunk) and the",
          "distillation target and loss passes over the same positions. Per launch, averaged over the",
          f"launches: the GPU's active cycles per XCD (GRBM_GUI_ACTIVE over {MI355X_XCDS} XCDs); resident",
          f"waves per SIMD (SQ_WAVE_CYCLES, in quad-cycles, over {MI355X_SIMDS} SIMDs and the active cycles);",
          "vector-ALU busy (SQ_ACTIVE_INST_VALU per CU over the active cycles: rocprofv3's VALUBusy); MFMA",
          "busy (SQ_VALU_MFMA_BUSY_CYCLES per SIMD over the active cycles: rocprofv3's MfmaUtil); the share",
          "of resident wave-cycles waiting on a dependency or a barrier (SQ_WAIT_ANY) and for issue",
          "(SQ_WAIT_INST_ANY); and the float32 transcendental instructions issued per launch.", "",
          "| kernel | launches | us (counter run) | active Mcycles per XCD | waves per SIMD | VALU busy % | MFMA busy % | waiting % | waiting for issue % | exp/log instructions (M) |",
          "|---|---:|---:|---:|---:|---:|---:|---:|---:|---:|"]
    for label, pat in SQ_KERNELS:
        ds = [d for (name, _), d in by.items() if pat in name and "GRBM_GUI_ACTIVE" in d]
        if not ds:
            continue

        def avg(key):
            return sum(d.get(key, 0.0) for d in ds) / len(ds)
        act = avg("GRBM_GUI_ACTIVE") / MI355X_XCDS
        wc = avg("SQ_WAVE_CYCLES")
        md.append(f"| `{label}` | {len(ds)} | {avg('_us'):.1f} | {act / 1e6:.3f} | "
                  f"{4 * wc / MI355X_SIMDS / act:.2f} | {400 * avg('SQ_ACTIVE_INST_VALU') / MI355X_SIMDS / act:.1f} | "
                  f"{100 * avg('SQ_VALU_MFMA_BUSY_CYCLES') / MI355X_SIMDS / act:.1f} | "
                  f"{100 * avg('SQ_WAIT_ANY') / wc:.1f} | {100 * avg('SQ_WAIT_INST_ANY') / wc:.1f} | "
                  f"{avg('SQ_INSTS_VALU_TRANS_F32') / 1e6:.1f} |")
    return "\n".join(md) + "\n"


def summarize_prefill_counters(mfma_dir: str, fetch_dir: str, write_dir: str, copy_mib: int = 1024) -> str:
    """MFMA and LDS utilisation and HBM traffic per launch of the prefill kernels (the causal
    indexer GEMM, the prefill attention, the per-row top-k) on the 8192-row prefill workload, from
    three rocprofv3 counter passes; FETCH_SIZE / WRITE_SIZE are scaled by what the same counters read
    for a plain device copy of copy_mib MiB."""
    import glob

    import clsa_synth as cs

    def rows(d):
        return _csv_rows(sorted(glob.glob(os.path.join(d, "*_counter_collection.csv")))[0])

    def per_kernel(rr, cname, pat):
        v = [float(r["Counter_Value"]) for r in rr if r["Counter_Name"] == cname and pat in r["Kernel_Name"]]
        return (sum(v) / len(v), len(v)) if v else (None, 0)

    m, f, wr = rows(mfma_dir), rows(fetch_dir), rows(write_dir)
    scale = {}
    for tag, rr, cname in (("fetch", f, "FETCH_SIZE"), ("write", wr, "WRITE_SIZE")):
        copy = max((r for r in rr if r["Counter_Name"] == cname and "copyBuffer" in r["Kernel_Name"]),
                   key=lambda r: int(r["Grid_Size"]))
        scale[tag] = (copy_mib * 1024.0) / float(copy["Counter_Value"])
    w = cs.config(4)
    n, L = w.n_rows, w.n_layers
    sel = sum(min(w.topk, t + 1) for t in range(n))
    alg_flop = {"k_index_scores_prefill": 2.0 * w.d_idx * n * (n + 1) / 2,
                "k_prefill_attn": 4.0 * sel * L * w.hq * w.head_dim}
    alg_bytes = {"k_index_scores_prefill": 2 * 2 * n * w.d_idx + 4 * n * (n + 1) // 2}
    md = ["# MFMA, LDS and HBM counters of the prefill kernels, prefill_n8k", "",
          "Made by (on one MI355X; each counter pass runs separately):", "",
          *[f"    {c}" for c in PREFILL_COUNTER_COMMANDS.values()],
          f"    python bench.py --summarize-prefill-counters {mfma_dir} {fetch_dir} {write_dir}", "",
          "The run holds warm-up and timed causal prefill steps of the 8192-row workload in one chunk of 8192 rows, then the",
          "indexer GEMM alone ten times. `MfmaUtil` is rocprofv3's derived percentage of the SIMDs' MFMA-busy",
          "cycles over the kernel's active cycles; `MfmaFlopsBF16` counts the bf16 MFMA work done (512 per",
          "MOPS); `LdsUtil` is the share of cycles the CUs' LDS is active; `LdsBankConflict` is conflicts per",
          f"access. FETCH_SIZE and WRITE_SIZE are scaled by a plain {copy_mib} MiB device copy in the same runs",
          f"(factors {scale['fetch']:.4f} and {scale['write']:.4f}).", "",
          "| kernel | launches | MfmaUtil % | MFMA TFLOP per launch | algorithmic TFLOP | LdsUtil % | LDS conflicts / access | HBM read MB | HBM write MB |",
          "|---|---:|---:|---:|---:|---:|---:|---:|---:|"]
    for label, pat in PREFILL_KERNELS:
        mu, cnt = per_kernel(m, "MfmaUtil", pat)
        fl, _ = per_kernel(m, "MfmaFlopsBF16", pat)
        lu, _ = per_kernel(m, "LdsUtil", pat)
        lb, _ = per_kernel(m, "LdsBankConflict", pat)
        fe, _ = per_kernel(f, "FETCH_SIZE", pat)
        wb, _ = per_kernel(wr, "WRITE_SIZE", pat)

        def fmt(x, k=2):
            return "-" if x is None else f"{x:.{k}f}"
        af = alg_flop.get(pat)
        md.append(f"| `{label}` | {cnt} | {fmt(mu)} | {fmt(None if fl is None else fl / 1e12, 4)} | "
                  f"{fmt(None if af is None else af / 1e12, 4)} | {fmt(lu)} | {fmt(lb, 4)} | "
                  f"{fmt(None if fe is None else fe * scale['fetch'] * 1024 / 1e6, 1)} | "
                  f"{fmt(None if wb is None else wb * scale['write'] * 1024 / 1e6, 1)} |")
    md += ["", f"Algorithmic bytes of the indexer GEMM: Q_idx and K_idx read once ({4 * n * w.d_idx / 1e6:.1f} MB) and the",
           f"causal fp32 scores written ({4 * n * (n + 1) // 2 / 1e6:.1f} MB), {alg_bytes['k_index_scores_prefill'] / 1e6:.1f} MB per launch."]
    return "\n".join(md) + "\n"


def trace_command(config: int) -> str:
    """The rocprofv3 kernel-trace command whose summary profiles/kernel_trace_<workload>.md holds."""
    if config == 4:
        return ("rocprofv3 --kernel-trace --stats --output-format csv -d rocprof_out/trace_prefill_n8k -o bench -- "
                "python3 bench.py --prefill-only --prefill-steps 3")
    import clsa_synth as cs
    tag = cs.config(config).name
    return (f"rocprofv3 --kernel-trace --stats --output-format csv -d rocprof_out/trace_{tag} -o bench -- "
            f"python3 bench.py --config {config} --steps 20 --warmup 3 {_DECODE_ONLY}")


def _csv_rows(path):
    import csv
    with open(path, newline="") as f:
        return list(csv.DictReader(f))


def _short_kernel(name: str) -> str:
    n = name.replace("(anonymous namespace)::", "").split("(")[0]
    for pre in ("void ", "clsa::", "at::native::"):
        n = n.replace(pre, "")
    return n.strip()


_TRACE_CONTENT = {
    "decode": ["The run holds warmup and timed steps of the layer-batched step (score kernel with histogram,",
               "top-k select, sparse attention), each preceded by the cache flush (a torch reduction over",
               "512 MiB), the same steps back to back, the score kernel alone (the roofline line), the",
               "per-layer schedule (gather + one attention per layer), the per-layer routing ablation",
               "(scores, top-k and one attention per layer), the new-token indexer projections and cache",
               "append ahead of the step, the Infinity Cache probes (torch reduce and copy) and the",
               "synthetic-input fill."],
    "prefill": ["The run holds warm-up and timed causal prefill steps (8192 rows in one chunk: the causal indexer GEMM, the",
                "per-row top-k, the sparse attention of every row over its own selection), the indexer GEMM",
                "alone, the distillation target and loss passes, and the synthetic-input fill."],
}


def summarize_trace(trace_dir: str, config: int = 3) -> tuple:
    """Markdown table of rocprofv3's kernel statistics (``*_kernel_stats.csv``); returns
    (workload tag, markdown)."""
    import glob

    import clsa_synth as cs
    tag = cs.config(config).name
    path = sorted(glob.glob(os.path.join(trace_dir, "*_kernel_stats.csv")))[0]
    kind = "prefill" if config == 4 else "decode"
    lines = [f"# Kernel trace: {kind} step, {tag}", "",
             "Made by (on one MI355X):", "", f"    {trace_command(config)}",
             f"    python bench.py --summarize-trace {trace_dir} --config {config}", "",
             *_TRACE_CONTENT[kind], "",
             "| kernel | calls | avg us | min us | max us | share % |", "|---|---:|---:|---:|---:|---:|"]
    for r in _csv_rows(path):
        lines.append(f"| `{_short_kernel(r['Name'])}` | {r['Calls']} | {float(r['AverageNs']) / 1e3:.2f} | "
                     f"{float(r['MinNs']) / 1e3:.2f} | {float(r['MaxNs']) / 1e3:.2f} | {float(r['Percentage']):.2f} |")
    # The decode score kernel's launches by kind: in the step (and the ablations) each launch is
    # followed by the top-k select; the scores-only launches run back to back (the roofline line)
    # or each after the cache flush.
    traces = sorted(glob.glob(os.path.join(trace_dir, "*_kernel_trace.csv")))
    if traces and kind == "decode":
        tr = sorted(_csv_rows(traces[0]), key=lambda r: int(r["Start_Timestamp"]))
        b2b, flushed, other = [], [], []
        for i, r in enumerate(tr):
            if "k_index_scores_decode" not in r["Kernel_Name"]:
                continue
            us = (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3
            if i + 1 < len(tr) and "k_topk" in tr[i + 1]["Kernel_Name"]:
                other.append(us)
            elif i > 0 and "reduce_kernel" in tr[i - 1]["Kernel_Name"]:
                flushed.append(us)
            else:
                b2b.append(us)
        lines += ["", "`k_index_scores_decode` by kind of launch (from the per-dispatch trace):", "",
                  "| launches | calls | avg us | min us | max us |", "|---|---:|---:|---:|---:|"]
        for name, v in (("scores only, back to back (the roofline line)", b2b),
                        ("scores only, each right after the cache flush", flushed),
                        ("followed by the top-k select (step, routing ablation, append)", other)):
            if v:
                lines.append(f"| {name} | {len(v)} | {sum(v) / len(v):.2f} | {min(v):.2f} | {max(v):.2f} |")
        # the layer-batched step's kernels, from the first kernel's start to the last one's end, per
        # kind of step; the bench runs those steps before its first scores-only launch
        first_alone = next((i for i, r in enumerate(tr) if "k_index_scores_decode" in r["Kernel_Name"] and not (
            i + 1 < len(tr) and "k_topk" in tr[i + 1]["Kernel_Name"])), len(tr))
        steps = {"after the cache flush": [], "back to back": []}
        for i in range(min(first_alone, len(tr)) - 2):
            if ("k_index_scores_decode" in tr[i]["Kernel_Name"] and "k_topk_select" in tr[i + 1]["Kernel_Name"]
                    and "k_sparse_attn" in tr[i + 2]["Kernel_Name"]):
                span = (int(tr[i + 2]["End_Timestamp"]) - int(tr[i]["Start_Timestamp"])) / 1e3
                fl = i > 0 and "reduce_kernel" in tr[i - 1]["Kernel_Name"]
                steps["after the cache flush" if fl else "back to back"].append(span)
        lines += ["", "The layer-batched step's three kernels, first start to last end:", "",
                  "| steps | calls | median us | min us | max us |", "|---|---:|---:|---:|---:|"]
        for name, v in steps.items():
            if v:
                lines.append(f"| {name} | {len(v)} | {float(np.median(v)):.2f} | {min(v):.2f} | {max(v):.2f} |")
    return tag, "\n".join(lines) + "\n"


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
    # the roofline's algorithmic bytes are the reads (K_idx + q_idx); the fp32 score write is an
    # intermediate, counted here on the write side
    alg_read = b["k_idx"] + b["q_idx"]
    score_write = 4 * w.total_tokens
    alg = alg_read + score_write
    fetch_b = out["fetch"]["kib_per_launch"] * out["fetch"]["scale"] * 1024.0
    write_b = out["write"]["kib_per_launch"] * out["write"]["scale"] * 1024.0
    rec = {"kernel": "k_index_scores_decode<128>", "workload": WORKLOAD_TAG, "kernel_source_sha": index_kernel_sha(),
           "kernel_sources": INDEX_KERNEL_SOURCES, "traffic_bytes_per_launch": round(traffic),
           "algorithmic_read_bytes_per_launch": alg_read, "score_write_bytes_per_launch": score_write,
           "fetch_over_algorithmic_read": round(fetch_b / alg_read, 4),
           "write_over_score_write": round(write_b / score_write, 4),
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
          f"scores written): {alg:,} B; ratio {traffic / alg:.4f}.",
          f"Reads: {fetch_b:,.0f} B against {alg_read:,} B of K_idx + q_idx (ratio {fetch_b / alg_read:.4f}; the",
          "roofline line counts these bytes). Writes: "
          f"{write_b:,.0f} B against {score_write:,} B of fp32 scores (ratio {write_b / score_write:.4f}).", "",
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
        return nbytes / ((ev0.elapsed_time(ev1) / 1e3) / 50) / 1e9

    read = rate(lambda: x.sum(), mib << 20)
    copy = rate(lambda: dst.copy_(half), mib << 20)
    return {"read_gbps": round(read, 1), "copy_gbps": round(copy, 1), "gbps": round(max(read, copy), 1)}


def hbm_stream_gbps(stream, read_mib: int = 2048, copy_mib: int = 1024) -> dict:
    """What plain streaming kernels reach from HBM on this machine, as a secondary yardstick for the
    step's algorithmic rate: a read-only reduction over read_mib MiB and a device copy of copy_mib
    MiB (read and write bytes counted), both larger than the 256 MB Infinity Cache."""
    import torch
    src = torch.ones(read_mib << 18, dtype=torch.float32, device="cuda")
    a = torch.ones(copy_mib << 18, dtype=torch.float32, device="cuda")
    b = torch.empty_like(a)

    def rate(fn, nbytes, reps=10):
        with torch.cuda.stream(stream):
            for _ in range(3):
                fn()
            ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            ev0.record(stream)
            for _ in range(reps):
                fn()
            ev1.record(stream)
        torch.cuda.synchronize()
        return nbytes / ((ev0.elapsed_time(ev1) / 1e3) / reps) / 1e9

    read = rate(lambda: src.sum(), read_mib << 20)
    copy = rate(lambda: b.copy_(a), 2 * (copy_mib << 20))
    del src, a, b
    torch.cuda.empty_cache()
    return {"read_mib": read_mib, "read_gbps": round(read, 1), "copy_mib": copy_mib, "copy_gbps": round(copy, 1),
            "gbps": round(max(read, copy), 1)}


def per_layer_bound(w, balg_total: float, ic_gbps: float) -> tuple:
    """The dependent-layer schedule's roofline: the step's algorithmic bytes from HBM at the peak,
    plus the compact K_S/V_S re-read once per layer at the rate measured for cache-resident data.
    Returns (bound seconds, compact bytes per layer)."""
    sel = sum(2 * w.hkv * min(w.topk, n) * w.head_dim * 2 for n in w.seq_lens)
    return balg_total / (HBM_PEAK_GBPS * 1e9) + w.n_layers * sel / (ic_gbps * 1e9), sel


def decode_configs_report(configs=(1, 2, 5), steps: int = 50, warmup: int = 10, flush=None, ic_gbps=None) -> dict:
    """The layer-batched decode step on the other decode workloads (the single short row, the
    32K batch, and the ragged 64-sequence batch with tie-heavy indexer entries), reported beside
    the 128K line: device time per step from HIP events around each step, with the caches flushed
    before every step (median, p10, p90) and back to back with no flush ("hot"), the host wall time
    per step of the hot loop, tokens/s and the algorithmic HBM rate against the 8 TB/s peak."""
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

        def one():
            clsa.step(dims, rows, dw.q_idx, dw.k_idx, dw.k_cache, dw.v_cache, dw.cu_seqlens, dw.q, out, idx, cnt,
                      ws, nws, stream=stream)

        for _ in range(warmup):
            one()
        cold, _ = event_times(stream, one, steps, flush=flush)
        hot, hot_wall = event_times(stream, one, steps)
        t = float(np.median(cold))
        b = algorithmic_bytes(w)["total"]
        per_layer = None
        if ic_gbps:
            nws2 = clsa.workspace_bytes(dims, rows, clsa.SCHEDULE_PER_LAYER)
            ws2 = torch.empty(nws2, dtype=torch.uint8, device="cuda")

            def one_pl():
                clsa.step(dims, rows, dw.q_idx, dw.k_idx, dw.k_cache, dw.v_cache, dw.cu_seqlens, dw.q, out, idx,
                          cnt, ws2, nws2, schedule=clsa.SCHEDULE_PER_LAYER, stream=stream)

            for _ in range(3):
                one_pl()
            pl, _ = event_times(stream, one_pl, max(10, steps // 5), flush=flush)
            t_pl = float(np.median(pl))
            bound, sel = per_layer_bound(w, b, ic_gbps)
            per_layer = {"ms_per_step": round(t_pl * 1e3, 4), "compact_bytes_per_layer": sel,
                         "bound_ms": round(bound * 1e3, 4), "frac": round(bound / t_pl, 4)}
            log(f"{w.name} per-layer schedule: {t_pl * 1e6:.1f} us (bound {bound * 1e6:.1f} us)")
            del ws2
        log(f"{w.name}: {t * 1e6:.1f} us flushed, {float(np.median(hot)) * 1e6:.1f} us hot")
        out_rep[w.name] = {"rows": R, "tokens": w.total_tokens, "max_row_len": w.max_row_len, "topk": k,
                           "layers": w.n_layers, "ms_per_step": round(t * 1e3, 4), "tokens_per_s": round(R / t, 1),
                           "bytes_alg_per_step": b, "hbm_gbps_alg": round(b / t / 1e9, 1),
                           "roofline_frac": round(b / t / 1e9 / HBM_PEAK_GBPS, 4),
                           "flushed": distribution(cold), "hot": distribution(hot),
                           "hot_wall_ms_per_step": round(hot_wall / steps * 1e3, 4),
                           "hot_roofline_frac": round(b / float(np.median(hot)) / 1e9 / HBM_PEAK_GBPS, 4),
                           "per_layer_schedule": per_layer}
        del dw, out, idx, cnt, ws
        torch.cuda.empty_cache()
    return out_rep


def prefill_report(steps: int = 8, chunk: int = 8192) -> dict:
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

    run(3)  # warm-up, as for the decode steps
    step_times, _ = event_times(stream, lambda: run(1), steps)
    t_step = float(np.median(step_times))
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    run(steps)
    torch.cuda.synchronize()
    t_wall = (time.perf_counter() - t0) / steps
    log(f"prefill step: median {t_step * 1e3:.3f} ms (events per step), {t_wall * 1e3:.3f} ms back to back (wall)")
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
    t_idx = (ev0.elapsed_time(ev1) / 1e3) / 10
    idx_flop = 2.0 * w.d_idx * (R * (R + 1) // 2)
    return {"workload": w.name, "rows": R, "topk": k, "layers": L, "chunk_rows": chunk, "steps": steps,
            "ms_per_step": round(t_step * 1e3, 3), "timing": distribution(step_times),
            "wall_ms_per_step_back_to_back": round(t_wall * 1e3, 3), "tokens_per_s": round(R / t_step, 1),
            "attn_tflops_alg": round(attn_flop / t_step / 1e12, 1),
            "attn_mfma_frac_of_step": round(attn_flop / t_step / 1e12 / MFMA_BF16_PEAK_TFLOPS, 4),
            "gather_bytes": gather_bytes, "gather_tbps": round(gather_bytes / t_step / 1e12, 2),
            "index_gemm_us": round(t_idx * 1e6, 1), "index_gemm_tflops": round(idx_flop / t_idx / 1e12, 1),
            "index_gemm_mfma_frac": round(idx_flop / t_idx / 1e12 / MFMA_BF16_PEAK_TFLOPS, 4)}


def distill_report(reps: int = 7) -> dict:
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

    run(2)
    times = []
    for _ in range(reps):  # each call timed on its own, the median reported
        ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        ev0.record(stream)
        run(1)
        ev1.record(stream)
        torch.cuda.synchronize()
        times.append(ev0.elapsed_time(ev1) / 1e3)
    times.sort()
    t = times[len(times) // 2]
    log(f"distillation: {t * 1e3:.3f} ms (min {times[0] * 1e3:.3f}, max {times[-1] * 1e3:.3f})")
    pairs = R * (R + 1) // 2                          # causal (position, key) pairs
    flop = 2 * pairs * L * hq * w.head_dim * 2         # two passes of q.k, 2 flop per MAC
    exps = 2 * pairs * L * hq                          # one exp2 per score and pass
    return {"workload": w.name, "rows": R, "layers": L, "heads": hq, "reps": reps, "ms": round(t * 1e3, 3),
            "ms_min": round(times[0] * 1e3, 3), "ms_max": round(times[-1] * 1e3, 3),
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

    # at most 16 threads: the host share that one GPU's box grants, whatever os.cpu_count() shows
    threads = max(1, min(16, os.cpu_count() or 1))
    one_rows, one_t = 0, 0.0
    while one_t < budget_s / 2 and one_rows < 4 * w.n_rows:
        _, t = C.oracle_rows_timed(w, [one_rows % w.n_rows], threads=1)
        one_t += t
        one_rows += 1
    log(f"oracle on one thread: {one_rows} rows in {one_t:.1f} s")
    all_rows, all_t = 0, 0.0
    while all_t < budget_s / 2:
        _, t = C.oracle_rows_timed(w, list(range(w.n_rows)), threads=threads)
        all_t += t
        all_rows += w.n_rows
    return {"value": round(all_rows / all_t, 2), "unit": "tokens/s", "cores": threads, "kind": "oracle",
            **host_cpu(), "one_core_tokens_per_s": round(one_rows / one_t, 3),
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
    ap.add_argument("--summarize-trace", metavar="DIR",
                    help="write the kernel-trace summary of --config's workload under profiles/ and exit")
    ap.add_argument("--summarize-prefill-counters", nargs=3, metavar=("MFMA_DIR", "FETCH_DIR", "WRITE_DIR"),
                    help="write the prefill kernels' counter summary under profiles/ and exit")
    ap.add_argument("--prefill-only", action="store_true",
                    help="run only the prefill report (and the distillation report unless --no-distill)")
    ap.add_argument("--prefill-steps", type=int, default=8)
    ap.add_argument("--summarize-sq-counters", metavar="DIR",
                    help="write the prefill and distillation kernels' issue and residency summary under profiles/ and exit")
    ap.add_argument("--summarize-counters", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"),
                    help="write the score kernel's HBM traffic summary under profiles/ and exit")
    args = ap.parse_args()
    if args.summarize_sq_counters:
        p = os.path.join(ROOT, "profiles", "counters_issue_prefill_distill_prefill_n8k.md")
        open(p, "w").write(summarize_sq_counters(args.summarize_sq_counters))
        print("wrote", p)
        return
    if args.summarize_prefill_counters:
        p = os.path.join(ROOT, "profiles", "counters_prefill_kernels_prefill_n8k.md")
        open(p, "w").write(summarize_prefill_counters(*args.summarize_prefill_counters))
        print("wrote", p)
        return
    if args.summarize_trace or args.summarize_counters:
        os.makedirs(os.path.join(ROOT, "profiles"), exist_ok=True)
        if args.summarize_trace:
            tag, md = summarize_trace(args.summarize_trace, args.config)
            p = os.path.join(ROOT, "profiles", f"kernel_trace_{tag}.md")
            open(p, "w").write(md)
            print("wrote", p)
        if args.summarize_counters:
            rec, md = summarize_counters(*args.summarize_counters)
            json.dump(rec, open(TRAFFIC_FILE, "w"), indent=1)
            p = os.path.join(ROOT, "profiles", f"hbm_traffic_index_scores_{WORKLOAD_TAG}.md")
            open(p, "w").write(md)
            print("wrote", TRAFFIC_FILE, "and", p)
        return
    if args.gpus != 1:
        print("bench.py runs on one GPU only: the library has no multi-GPU path (use --gpus 1)", file=sys.stderr)
        sys.exit(2)

    import torch

    import clsa_synth as cs
    import cross_layer_token_amd as clsa
    from clsa_synth.device import DeviceWorkload

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    if args.prefill_only:
        rep = {"prefill": prefill_report(steps=args.prefill_steps)}
        if not args.no_distill:
            rep["distill"] = distill_report()
        if args.profile_copy_mib > 0:
            src = torch.ones(args.profile_copy_mib << 20, dtype=torch.uint8, device="cuda")
            dst = torch.empty_like(src)
            dst.copy_(src)
            torch.cuda.synchronize()
        print(json.dumps(rep), flush=True)
        return
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
        return (ev0.elapsed_time(ev1) / 1e3), wall

    flush = Flush(stream)

    # ---- the step (layer-batched schedule) ------------------------------------------------------
    # Timed protocol: HIP events around every step, the caches flushed before each step outside
    # its events (so neither K_idx nor the selected K/V rows of the previous step are cache-resident
    # when a step starts); value and ms_per_step are the median over the steps.  The same steps back
    # to back with no flush are reported beside it.
    nws = clsa.workspace_bytes(dims, rows, clsa.SCHEDULE_LAYER_BATCHED)
    ws = torch.empty(nws, dtype=torch.uint8, device="cuda")
    run_steps(args.warmup, clsa.SCHEDULE_LAYER_BATCHED, ws, nws)
    step_times, step_wall = event_times(stream, lambda: run_steps(1, clsa.SCHEDULE_LAYER_BATCHED, ws, nws),
                                        args.steps, flush=flush)
    t_step = float(np.median(step_times))
    t_gpu_hot, t_wall_hot = timed(lambda n: run_steps(n, clsa.SCHEDULE_LAYER_BATCHED, ws, nws), args.steps)
    hot_times, _ = event_times(stream, lambda: run_steps(1, clsa.SCHEDULE_LAYER_BATCHED, ws, nws), args.steps)
    balg = algorithmic_bytes(w)
    hbm_gbps = balg["total"] / t_step / 1e9
    log(f"{w.name} step: median {t_step * 1e6:.1f} us flushed, {float(np.median(hot_times)) * 1e6:.1f} us hot")

    # ---- the dominant kernel alone: routing scores streamed from K_idx --------------------------
    # Its algorithmic bytes are the K_idx scan and the queries; the fp32 score write is an
    # intermediate of the method and is reported separately.  The launch time is the mean over
    # launches back to back between one pair of events: K_idx (512 MiB, streamed with non-temporal
    # loads) is larger than the Infinity Cache, so no launch finds the previous one's bytes cached,
    # and a kernel recorded alone between two events starts about 5.5 us after its start event
    # (the event's completion handshake; see the kernel trace), which would be counted as kernel
    # time.  Per-launch events with the flush before each launch are reported beside it.
    ld = ((w.max_row_len + 63) // 64) * 64
    scores = torch.empty((R, ld), dtype=torch.float32, device="cuda")

    def run_scores(n):
        for _ in range(n):
            clsa.index_scores(dims, rows, dw.q_idx, dw.k_idx, dw.cu_seqlens, scores, ld, stream=stream)

    run_scores(args.warmup)
    t_idx_all, _ = timed(run_scores, args.steps)
    t_idx = t_idx_all / args.steps
    idx_times, _ = event_times(stream, lambda: run_scores(1), args.steps, flush=flush)
    idx_bytes = balg["k_idx"] + balg["q_idx"]          # K_idx + q_idx read
    achieved = idx_bytes / t_idx / 1e9
    roofline = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                "frac": round(achieved / HBM_PEAK_GBPS, 4), "traffic": measured_traffic(idx_bytes),
                "kernel": "k_index_scores_decode<128>", "bytes_per_launch": idx_bytes,
                "score_write_bytes_per_launch": 4 * w.total_tokens, "us_per_launch": round(t_idx * 1e6, 2),
                "launches": args.steps,
                "flushed_per_launch_events_us": {k2.replace("_ms", ""): (round(v * 1e3, 2) if k2.endswith("_ms") else v)
                                                 for k2, v in distribution(idx_times).items()},
                "with_score_write_frac": round((idx_bytes + 4 * w.total_tokens) / t_idx / 1e9 / HBM_PEAK_GBPS, 4)}
    flush_check = cache_flush_check(stream, flush)
    log(f"score kernel alone: {t_idx * 1e6:.2f} us per launch; flush check {flush_check}")

    # ---- dependent-layer schedule (one attention pass per layer), reported beside -----------------
    per_layer = None
    if not args.no_per_layer:
        nws2 = clsa.workspace_bytes(dims, rows, clsa.SCHEDULE_PER_LAYER)
        ws2 = torch.empty(nws2, dtype=torch.uint8, device="cuda")
        run_steps(args.warmup, clsa.SCHEDULE_PER_LAYER, ws2, nws2)
        pl_times, _ = event_times(stream, lambda: run_steps(1, clsa.SCHEDULE_PER_LAYER, ws2, nws2), args.steps,
                                  flush=flush)
        t_pl = float(np.median(pl_times))
        # its roofline: the step's algorithmic bytes from HBM, plus the compact K_S/V_S read once
        # per layer from the Infinity Cache, at the rate a cache-resident device copy reaches here
        ic = infinity_cache_gbps(stream)
        bound, sel_bytes = per_layer_bound(w, balg["total"], ic["gbps"])
        log(f"per-layer schedule: {t_pl * 1e6:.1f} us")
        per_layer = {"ms_per_step": round(t_pl * 1e3, 4), "tokens_per_s": round(R / t_pl, 1),
                     "timing": distribution(pl_times),
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
        r_times, _ = event_times(stream, lambda: run_routing(1), n3, flush=flush)
        t3 = float(np.median(r_times))
        log(f"per-layer routing: {t3 * 1e6:.1f} us")
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
        a_times, _ = event_times(stream, lambda: run_append_steps(1), args.steps, flush=flush)
        t4 = float(np.median(a_times))
        # the projection's cost is what it adds to the (device-bound) step; timing the kernel alone
        # from back-to-back host calls would measure the host's call rate instead
        added = t4 - t_step
        log(f"append + step: {t4 * 1e6:.1f} us")
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
    stream_bw = hbm_stream_gbps(stream)
    log(f"HBM stream rates measured here: {stream_bw}")
    decode_configs = None if args.no_decode_configs else decode_configs_report(
        flush=flush, ic_gbps=per_layer["roofline"]["infinity_cache"]["gbps"] if per_layer else None)
    prefill = None if args.no_prefill else prefill_report()
    distill = None if args.no_distill else distill_report()
    cpu = None if args.no_cpu_baseline else cpu_baseline(w, args.cpu_budget)
    line = {
        "metric": METRIC,
        "value": round(R / t_step, 1),
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
        "hbm_stream": stream_bw,
        "step_frac_of_measured_stream": round(hbm_gbps / stream_bw["gbps"], 4),
        "bytes_alg_per_step": balg["total"],
        "step_timing": {"protocol": f"HIP events around each step; a {FLUSH_MIB} MiB read before every step, outside "
                                    "its events; median over the steps (the step's first kernel starts about 5.5 us "
                                    "after its start event, which this figure counts)",
                        "flushed": distribution(step_times), "flushed_wall_s": round(step_wall, 3),
                        "hot": distribution(hot_times),
                        "hot_back_to_back_ms_per_step": round(t_gpu_hot / args.steps * 1e3, 4),
                        "hot_wall_ms_per_step": round(t_wall_hot / args.steps * 1e3, 4),
                        "hot_roofline_frac": round(balg["total"] / (t_gpu_hot / args.steps) / 1e9 / HBM_PEAK_GBPS, 4),
                        "cache_flush_check": flush_check},
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
