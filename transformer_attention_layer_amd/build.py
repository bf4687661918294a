"""Compile the HIP sources of the GQA layer into ``libgqa.so`` (gfx950), the
measurement microkernels into ``libgqa_peaks.so``, and the same layer
sources with ``GQA_LDS_POISON`` into ``libgqa_ldspoison.so``: a debug build
whose kernels first fill their LDS with NaN bits, which a GPU test runs the
parity checks against (a read of LDS that nothing wrote then shows up).

Run ``python -m transformer_attention_layer_amd.build`` or call ``build()``.
Every source is compiled with hipcc for gfx950 only; packed fp32 VALU forms
are disabled (``-packed-fp32-ops``), and the objects are linked into shared
libraries next to this file.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
BUILD_DIR = os.path.join(os.path.dirname(HERE), "_build")
LIB = os.path.join(HERE, "libgqa.so")
SOURCES = ["gqa_api.hip", "gemm_bf16.hip", "attn_bf16.hip", "attn_bwd.hip", "bwd_kernels.hip",
           "normrope_rows.hip", "f32_kernels.hip"]
PEAKS_LIB = os.path.join(HERE, "libgqa_peaks.so")
PEAKS_SOURCES = ["peaks.hip"]
POISON_LIB = os.path.join(HERE, "libgqa_ldspoison.so")
POISON_DIR = os.path.join(BUILD_DIR, "ldspoison")

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"
FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-Wall",
    "-Wno-unused-function",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
]


def _compile(job) -> str:
    src, poison = job
    obj = os.path.join(POISON_DIR if poison else BUILD_DIR, os.path.splitext(src)[0] + ".o")
    cmd = [HIPCC, *FLAGS, *(["-DGQA_LDS_POISON"] if poison else []), "-c",
           os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    return obj


def _link(objs, lib: str) -> None:
    tmp = lib + ".tmp"
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, lib)


def build(verbose: bool = False) -> str:
    """Compile every source, link ``libgqa.so``, ``libgqa_peaks.so`` and
    ``libgqa_ldspoison.so``; returns the layer library's path."""
    os.makedirs(BUILD_DIR, exist_ok=True)
    os.makedirs(POISON_DIR, exist_ok=True)
    jobs = [(s, False) for s in SOURCES + PEAKS_SOURCES] + [(s, True) for s in SOURCES]
    with cf.ThreadPoolExecutor(max_workers=min(len(jobs), os.cpu_count() or 1)) as ex:
        objs = list(ex.map(_compile, jobs))
    n, m = len(SOURCES), len(PEAKS_SOURCES)
    _link(objs[:n], LIB)
    _link(objs[n:n + m], PEAKS_LIB)
    _link(objs[n + m:], POISON_LIB)
    if verbose:
        print(f"built {LIB}, {PEAKS_LIB} and {POISON_LIB}")
    return LIB


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
