"""Build the HIP libraries in-tree for gfx950.

    python -m cross_layer_token_amd.build

produces ``cross_layer_token_amd/libclsa.so`` (the CLSA C ABI of include/clsa.h) and
``clsa_synth/libclsa_synth.so`` (the device filler of the synthetic inputs).
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PKG = os.path.join(ROOT, "cross_layer_token_amd")
CSRC = os.path.join(PKG, "csrc")
SYNTH = os.path.join(ROOT, "clsa_synth")
BUILD = os.path.join(ROOT, "_build")

ARCH = "gfx950"
# Packed fp32 instructions are kept off for every HIP translation unit.
# Code object v5 loads under both the ROCm runtime in /opt/rocm and the one bundled with torch.
HIPFLAGS = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}", "-mcode-object-version=5", "-Wall",
            "-Wno-unused-function",
            "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]
LIB_SOURCES = ["plan.cpp", "api.cpp", "k_index.hip", "k_topk.hip", "k_attn.hip", "k_project.hip", "k_distill.hip",
               "no_alloc.hip"]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found")


def _run(cmd):
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    out = "\n".join(l for l in r.stdout.splitlines() if "packed-fp32-ops" not in l and "1 warning generated" not in l)
    if r.returncode != 0:
        raise RuntimeError(f"build failed: {' '.join(cmd)}\n{out}")
    return out


def _compile(src: str, obj: str) -> str:
    lang = ["-x", "hip"] if src.endswith(".hip") else []
    return _run([hipcc()] + HIPFLAGS + lang + ["-c", src, "-o", obj])


def build(verbose: bool = False) -> list:
    os.makedirs(BUILD, exist_ok=True)
    jobs = [(os.path.join(CSRC, s), os.path.join(BUILD, s + ".o")) for s in LIB_SOURCES]
    jobs.append((os.path.join(SYNTH, "synth.hip"), os.path.join(BUILD, "synth.hip.o")))
    with ThreadPoolExecutor(max_workers=min(8, len(jobs))) as ex:
        logs = list(ex.map(lambda j: _compile(*j), jobs))
    lib = os.path.join(PKG, "libclsa.so")
    synth = os.path.join(SYNTH, "libclsa_synth.so")
    _run([hipcc(), "-shared", "-fPIC", f"--offload-arch={ARCH}"] + [o for _, o in jobs[:-1]] + ["-o", lib + ".tmp"])
    os.replace(lib + ".tmp", lib)
    _run([hipcc(), "-shared", "-fPIC", f"--offload-arch={ARCH}", jobs[-1][1], "-o", synth + ".tmp"])
    os.replace(synth + ".tmp", synth)
    if verbose:
        for l in logs:
            if l.strip():
                print(l)
    return [lib, synth]


if __name__ == "__main__":
    for p in build(verbose="-v" in sys.argv):
        print("built", p)
