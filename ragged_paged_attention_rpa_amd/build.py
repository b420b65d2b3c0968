"""Builds librpa.so (the HIP/gfx950 kernels and the C ABI) in-tree with hipcc.

Usage: python -m ragged_paged_attention_rpa_amd.build  [--jobs N]
"""
from __future__ import annotations

import argparse
import concurrent.futures as cf
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
ROOT = os.path.dirname(HERE)
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(HERE, "librpa.so")
ARCH = "gfx950"

SOURCES = ["rpa_api.cpp", "tile_table.cpp", "kv_update.hip", "gqa_attn.hip", "gqa_prefill.hip",
           "mla_attn.hip", "mla_decode.hip", "probes.hip"]

# Packed-fp32 VALU ops stay off: the compiler must not emit v_pk_{add,mul,fma}_f32.
HIPCC_FLAGS = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
               "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
               "-Wall", "-Wno-unused-function", "-I", os.path.join(ROOT, "include")]


def _hipcc():
    return os.path.join(os.environ.get("ROCM_PATH", "/opt/rocm"), "bin", "hipcc")


# Per-file flags. mla_decode.hip keeps its QK^T accumulators in VGPRs (the
# MFMA "VGPR form"): its 256 AGPRs hold the output accumulators.
FILE_FLAGS = {"mla_decode.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"]}


def _compile(src):
    os.makedirs(BUILD, exist_ok=True)
    obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
    cmd = [_hipcc(), *HIPCC_FLAGS, *FILE_FLAGS.get(src, []), "-x", "hip", "-c",
           os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stdout}\n{r.stderr}")
    warn = "\n".join(l for l in r.stderr.splitlines()
                     if "packed-fp32-ops" not in l and l.strip())
    return obj, warn


def build(jobs: int = 8, verbose: bool = False) -> str:
    """Compiles every source for gfx950 and links librpa.so; returns its path."""
    with cf.ThreadPoolExecutor(max_workers=max(1, jobs)) as ex:
        results = list(ex.map(_compile, SOURCES))
    objs = [o for o, _ in results]
    if verbose:
        for (o, w) in results:
            if w:
                print(w, file=sys.stderr)
    tmp = LIB + ".tmp%d" % os.getpid()
    rocm_lib = os.path.join(os.environ.get("ROCM_PATH", "/opt/rocm"), "lib")
    cmd = [_hipcc(), "-shared", "-fPIC", f"--offload-arch={ARCH}", "-o", tmp, *objs,
           "-L", rocm_lib, "-lrocprofiler-sdk-roctx", "-Wl,-rpath," + rocm_lib]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    ap = argparse.ArgumentParser()
    ap.add_argument("--jobs", type=int, default=8)
    ap.add_argument("-v", "--verbose", action="store_true")
    args = ap.parse_args()
    print(build(args.jobs, args.verbose))
