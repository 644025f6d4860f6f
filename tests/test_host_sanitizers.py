"""Host code of libpagedkv under AddressSanitizer and UndefinedBehaviorSanitizer (CPU only).

* the block pool (pkv_block_pool.cpp) built with g++ and driven through random
  operation streams with its invariants checked after every step;
* the C ABI's host layer (pkv_api.hip: argument checks, geometry, workspace sizes, split
  set-up) built with hipcc -- sanitizers on the host side only -- against stub kernel
  launchers, and called two million times with edge-case and random arguments.

Any sanitizer report aborts the driver, which fails the test."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HERE = os.path.join(ROOT, "tests", "host_sanitize")
CSRC = os.path.join(ROOT, "paged_kv_cache_79_amd", "csrc")
INC = os.path.join(ROOT, "include")
ROCM_INC = "/opt/rocm/include"
HIPCC = "/opt/rocm/bin/hipcc"


def _no_gpu():
    import torch
    return not torch.cuda.is_available()


# the API driver hands dummy device pointers to the library; its launchers are stubs,
# but on a machine with a GPU the runtime would be live: CPU-only
cpu_only = pytest.mark.skipif(not _no_gpu(), reason="dummy device pointers: CPU-only test")


def _run(cmd, **kw):
    r = subprocess.run(cmd, capture_output=True, text=True, **kw)
    assert r.returncode == 0, f"{' '.join(cmd)}\n{r.stdout[-2000:]}\n{r.stderr[-4000:]}"
    return r.stdout


@pytest.mark.skipif(shutil.which("g++") is None, reason="g++ missing")
def test_block_pool_under_asan_ubsan(tmp_path):
    exe = str(tmp_path / "pool_driver")
    _run(["g++", "-std=c++17", "-O1", "-g", "-fno-omit-frame-pointer", "-D__HIP_PLATFORM_AMD__",
          "-fsanitize=address,undefined", "-fno-sanitize-recover=all", f"-I{INC}", f"-I{ROCM_INC}",
          os.path.join(HERE, "pool_driver.cpp"), os.path.join(CSRC, "pkv_block_pool.cpp"), "-o", exe])
    out = _run([exe], timeout=300)
    assert "invariants held" in out


@cpu_only
@pytest.mark.skipif(not os.path.exists(HIPCC), reason="hipcc missing")
def test_api_host_layer_under_asan_ubsan(tmp_path):
    exe = str(tmp_path / "api_driver")
    _run([HIPCC, "--offload-arch=gfx950", "-x", "hip", "-std=c++17", "-O1", "-g",
          "-fno-omit-frame-pointer", "-Wno-unused-command-line-argument",
          "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
          "-Xarch_host", "-fno-sanitize-recover=all", f"-I{INC}", f"-I{CSRC}",
          os.path.join(CSRC, "pkv_api.hip"), os.path.join(HERE, "launch_stubs.cpp"),
          os.path.join(HERE, "api_driver.cpp"), "-o", exe])
    out = _run([exe], timeout=300)
    assert "api calls:" in out
