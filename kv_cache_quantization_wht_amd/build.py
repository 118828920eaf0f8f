"""Build ``libtq.so`` in-tree with hipcc for gfx950.

Usage: ``python -m kv_cache_quantization_wht_amd.build`` (or ``__graft_entry__.build()``).
Objects go to ``_build/`` at the repository root; the shared library is written next to this file.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
OUT = os.path.join(HERE, "libtq.so")
BUILD = os.path.join(ROOT, "_build")

HIPCC = os.environ.get("HIPCC", shutil.which("hipcc") or "/opt/rocm/bin/hipcc")
ARCH = "gfx950"
COMMON = [
    "-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
    "-I", os.path.join(ROOT, "include"),
    # packed fp32 VALU forms are disabled; none of the kernels relies on them
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-unused-command-line-argument",
]
# (source, object, extra flags). The decode source is compiled in four parts (head_dim 128 / 64, each
# with packed or one-per-head query columns) so its kernel instantiations build in parallel. No NaN reaches
# a max or compare on the decode path (masked scores are finite), so the NaN-quieting copies in front of
# every max are dropped there. The head_dim 128 packed-column part (the kernels of every benchmarked
# workload) uses the instruction-level-parallelism scheduling strategy: measured 1-2% faster on the
# Llama-70B K4/V2 scan, neutral on the other workloads, no spills in the kernels they run.
SOURCES = [
    ("tq_capi.cpp", "tq_capi.o", []),
    ("tq_quantize.hip", "tq_quantize.o", []),
    ("tq_dense.hip", "tq_dense.o", ["-fno-honor-nans"]),
    ("tq_rotate.hip", "tq_rotate.o", []),
    ("tq_stream.hip", "tq_stream.o", []),
    ("tq_qr.cpp", "tq_qr.o", []),
    ("tq_prefill.hip", "tq_prefill.o", ["-fno-honor-nans"]),
    ("tq_decode.hip", "tq_decode_d128_pk.o",
     ["-fno-honor-nans", "-DTQ_DECODE_PART=1", "-mllvm", "-amdgpu-sched-strategy=max-ilp"]),
    ("tq_decode.hip", "tq_decode_d128.o", ["-fno-honor-nans", "-DTQ_DECODE_PART=2"]),
    ("tq_decode.hip", "tq_decode_d64_pk.o", ["-fno-honor-nans", "-DTQ_DECODE_PART=3"]),
    ("tq_decode.hip", "tq_decode_d64.o", ["-fno-honor-nans", "-DTQ_DECODE_PART=4"]),
]


def _compile(entry) -> str:
    src, obj_name, extra = entry
    obj = os.path.join(BUILD, obj_name)
    cmd = [HIPCC, *COMMON, *extra, "-c", os.path.join(CSRC, src), "-o", obj]
    if src.endswith(".hip"):
        cmd[1:1] = ["-x", "hip"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    return obj


def build(verbose: bool = True) -> str:
    os.makedirs(BUILD, exist_ok=True)
    with cf.ThreadPoolExecutor(max_workers=min(len(SOURCES), os.cpu_count() or 4)) as ex:
        objs = list(ex.map(_compile, SOURCES))
    tmp = OUT + ".tmp"
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, OUT)
    if verbose:
        print(f"built {OUT}")
    return OUT


if __name__ == "__main__":
    build()
    sys.exit(0)
