"""Build libpagedkv.so for gfx950 in-tree with hipcc.

    python -m paged_kv_cache_79_amd.build        # or paged_kv_cache_79_amd.build.build_library()

Objects go to ``_build/`` at the repository root; the shared library lands next
to this file so the binding (and a copy of the tree on another machine) finds it.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
OBJDIR = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libpagedkv.so")
# the benchmark's streaming-read ceiling kernel, kept out of libpagedkv's interface
BENCH_LIB = os.path.join(PKG, "libpkvbench.so")
BENCH_SOURCES = ["pkv_read_ceiling.hip"]
ARCH = "gfx950"

SOURCES = ["pkv_api.hip", "pkv_write_copy.hip", "pkv_decode.hip", "pkv_prefill.hip",
           "pkv_prefix.hip", "pkv_decode_mq.hip", "pkv_validate.hip",
           "pkv_block_pool.cpp"]

HIPCC_FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
    # packed fp32 ops stay off (v_pk_fma_f32 and friends are not emitted)
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-unused-command-line-argument",
    f"-I{INCLUDE}", f"-I{CSRC}",
]


def _hipcc() -> str:
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", "hipcc"):
        if c and (os.path.isabs(c) and os.path.exists(c) or not os.path.isabs(c)):
            return c
    return "hipcc"


def _compile(src: str) -> str:
    obj = os.path.join(OBJDIR, os.path.splitext(src)[0] + ".o")
    cmd = [_hipcc(), *HIPCC_FLAGS, "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{' '.join(cmd)}\n{r.stderr}")
    return obj


def _link(objs, out: str) -> None:
    tmp = out + ".tmp"
    cmd = [_hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{' '.join(cmd)}\n{r.stderr}")
    os.replace(tmp, out)


def build_library(verbose: bool = False) -> str:
    """Compile every HIP source, link libpagedkv.so (and the benchmark's
    libpkvbench.so); returns the libpagedkv path."""
    os.makedirs(OBJDIR, exist_ok=True)
    srcs = SOURCES + BENCH_SOURCES
    with cf.ThreadPoolExecutor(max_workers=min(len(srcs), os.cpu_count() or 4)) as ex:
        objs = list(ex.map(_compile, srcs))
    _link(objs[:len(SOURCES)], LIB)
    _link(objs[len(SOURCES):], BENCH_LIB)
    if verbose:
        print(f"built {LIB}")
        print(f"built {BENCH_LIB}")
    return LIB


if __name__ == "__main__":
    build_library(verbose=True)
    sys.exit(0)
