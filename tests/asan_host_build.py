"""Builds librpa with AddressSanitizer on its host code (the kernels are
compiled as usual): every source with the in-tree flags plus
-Xarch_host -fsanitize=address, linked against the shared sanitizer runtime.
Used by test_host_asan.py only (CPU side; nothing here runs on a GPU)."""
from __future__ import annotations

import concurrent.futures as cf
import os
import subprocess

from ragged_paged_attention_rpa_amd import build as B

OUT_DIR = os.path.join(B.ROOT, "_build", "asan")
LIB = os.path.join(OUT_DIR, "librpa_asan.so")
SAN_COMPILE = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fno-omit-frame-pointer"]
SAN_LINK = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-shared-libasan"]


def runtime() -> str:
    """Path of the shared sanitizer runtime the test preloads."""
    clang = os.path.join(os.environ.get("ROCM_PATH", "/opt/rocm"), "llvm", "bin", "clang++")
    r = subprocess.run([clang, "-print-file-name=libclang_rt.asan-x86_64.so"], capture_output=True,
                       text=True, check=True)
    return r.stdout.strip()


def _compile(src: str) -> str:
    obj = os.path.join(OUT_DIR, os.path.splitext(src)[0] + ".o")
    cmd = [B._hipcc(), *B.HIPCC_FLAGS, *SAN_COMPILE, *B.FILE_FLAGS.get(src, []), "-x", "hip", "-c",
           os.path.join(B.CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stderr}")
    return obj


def build(jobs: int = 8) -> str:
    os.makedirs(OUT_DIR, exist_ok=True)
    with cf.ThreadPoolExecutor(max_workers=jobs) as ex:
        objs = list(ex.map(_compile, B.SOURCES))
    rocm_lib = os.path.join(os.environ.get("ROCM_PATH", "/opt/rocm"), "lib")
    cmd = [B._hipcc(), "-shared", "-fPIC", f"--offload-arch={B.ARCH}", *SAN_LINK, "-o", LIB, *objs,
           "-L", rocm_lib, "-lrocprofiler-sdk-roctx", "-Wl,-rpath," + rocm_lib]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr}")
    return LIB
