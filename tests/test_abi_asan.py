"""The C ABI's host code under AddressSanitizer (CPU only).

api.hip (argument validation, error messages, size queries) is compiled with
host-side ASan and linked with the library's other objects into a small
driver, tests/asan/abi_driver.cpp, that walks every validation path of every
entry point. Validation returns before any HIP call, so no GPU is needed.
"""

import os
import shutil
import subprocess

import pytest

from tests.conftest import ROOT

CSRC = os.path.join(ROOT, "attention_paged_kv_cache_amd", "csrc")
BUILD = os.path.join(ROOT, "_build")
CLANG = "/opt/rocm/llvm/bin/clang++"


def run(cmd, **kw):
    r = subprocess.run(cmd, capture_output=True, text=True, timeout=600, **kw)
    assert r.returncode == 0, f"{' '.join(cmd)}\n{r.stdout}\n{r.stderr}"
    return r


def test_c_abi_host_code_under_asan(tmp_path):
    hipcc = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(hipcc) or not os.path.exists(CLANG):
        pytest.fail("ROCm toolchain not found")
    objs = [os.path.join(BUILD, f"{n}.hip.o") for n in ("append", "decode", "prefill")]
    if not all(os.path.exists(o) for o in objs):
        pytest.fail("library objects missing: run __graft_entry__.build() first")
    inc = [f"-I{os.path.join(ROOT, 'include')}", f"-I{CSRC}"]
    api_o, drv_o, exe = (str(tmp_path / n) for n in ("api_asan.o", "driver.o", "abi_asan"))
    run([hipcc, "--offload-arch=gfx950", "-O1", "-g", "-std=c++17", "-fPIC",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-Xarch_host", "-fsanitize=address", *inc, "-c", os.path.join(CSRC, "api.hip"),
         "-o", api_o])
    run([CLANG, "-O1", "-g", "-std=c++17", "-fsanitize=address", *inc, "-c",
         os.path.join(ROOT, "tests", "asan", "abi_driver.cpp"), "-o", drv_o])
    run([CLANG, "-fsanitize=address", drv_o, api_o, *objs, "-L/opt/rocm/lib", "-lamdhip64",
         "-Wl,-rpath,/opt/rocm/lib", "-o", exe])
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=0")
    r = subprocess.run([exe], capture_output=True, text=True, timeout=120, env=env)
    out = r.stdout + r.stderr
    assert "AddressSanitizer" not in out, out
    assert r.returncode == 0, out
    assert "ok (0 failures)" in r.stdout
