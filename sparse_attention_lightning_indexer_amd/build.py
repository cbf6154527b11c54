"""Build the HIP library ``libindexer.so`` in-tree for gfx950 with hipcc.

Run as ``python -m sparse_attention_lightning_indexer_amd.build``.  Each
source is compiled to an object under ``_build/`` (in parallel), then linked
into ``sparse_attention_lightning_indexer_amd/libindexer.so`` (the indexer's
C-ABI).  The measured-peak probes the benchmark reports beside the published
peaks are linked into a separate ``libpeak_probe.so``, outside the indexer's
ABI.
"""
from __future__ import annotations

import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libindexer.so")
SOURCES = ["indexer_api.hip", "score_kernel.hip", "decode_kernel.hip", "topk_kernel.hip", "pool_kernel.hip", "stream_topk.hip"]
PROBE_SOURCES = ["peak_probe.hip"]
PROBE_LIB = os.path.join(PKG, "libpeak_probe.so")
ARCH = os.environ.get("INDEXER_OFFLOAD_ARCH", "gfx950")

FLAGS = [
    "-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
    # keep the compiler from forming packed fp32 VALU ops
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-command-line-argument",
    "-I", os.path.join(ROOT, "include"),
]


def hipcc() -> str:
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    cand = os.path.join(rocm, "bin", "hipcc")
    return cand if os.path.exists(cand) else "hipcc"


def _compile(src: str) -> str:
    obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
    cmd = [hipcc(), *FLAGS, "-c", os.path.join(CSRC, src), "-o", obj]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{res.stdout}\n{res.stderr}")
    return obj


def _link(objs, out):
    tmp = out + ".tmp"
    cmd = [hipcc(), "-shared", "-fPIC", f"--offload-arch={ARCH}", "-o", tmp, *objs]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"link failed:\n{res.stdout}\n{res.stderr}")
    os.replace(tmp, out)


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    srcs = SOURCES + PROBE_SOURCES
    with ThreadPoolExecutor(max_workers=len(srcs)) as ex:
        objs = list(ex.map(_compile, srcs))
    _link(objs[: len(SOURCES)], LIB)
    _link(objs[len(SOURCES):], PROBE_LIB)
    if verbose:
        print(f"built {LIB} and {PROBE_LIB}")
    return LIB


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
