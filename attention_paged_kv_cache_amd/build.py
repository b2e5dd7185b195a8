"""Build libpkv.so (the HIP kernels and their C ABI) for gfx950 with hipcc,
and libpkv_ceiling.so (the chip-ceiling kernels the benchmark reads rates
against; no part of the attention path).

Run as ``python -m attention_paged_kv_cache_amd.build`` or through
``__graft_entry__.build()``. Objects go to ``_build/`` at the repository root;
the shared libraries land next to this file, where the binding loads them.
"""

import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
OUT = os.path.join(PKG, "libpkv.so")
CEILING_SRC = os.path.join(CSRC, "ceiling", "ceiling.hip")
CEILING_OUT = os.path.join(PKG, "libpkv_ceiling.so")
BUILD = os.path.join(ROOT, "_build")

ARCH = "gfx950"

# -Xclang -target-feature -Xclang -packed-fp32-ops: no packed fp32 VALU ops
# (v_pk_fma_f32 and friends) are generated.
HIPCC_FLAGS = [
    f"--offload-arch={ARCH}",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-fvisibility=hidden",
    "-Wall",
    "-Wno-unused-function",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    f"-I{INCLUDE}",
    f"-I{CSRC}",
]


def hipcc():
    path = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(path):
        raise RuntimeError("hipcc not found (ROCm is required to build libpkv.so)")
    return path


def sources():
    return sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC) if f.endswith(".hip"))


def _compile(src, verbose):
    obj = os.path.join(BUILD, os.path.basename(src) + ".o")
    cmd = [hipcc(), *HIPCC_FLAGS, "-c", src, "-o", obj]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{r.stdout}\n{r.stderr}")
    if r.stderr.strip() and verbose:
        print(r.stderr, file=sys.stderr)
    return obj


def _link(objs, out, verbose):
    tmp = out + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, out)


def build(verbose=False, jobs=None):
    """Compile every .hip source and link libpkv.so and libpkv_ceiling.so.
    Always rebuilds."""
    os.makedirs(BUILD, exist_ok=True)
    srcs = sources() + [CEILING_SRC]
    jobs = jobs or min(len(srcs), os.cpu_count() or 4, 8)
    with ThreadPoolExecutor(max_workers=jobs) as ex:
        objs = list(ex.map(lambda s: _compile(s, verbose), srcs))
    _link(objs[:-1], OUT, verbose)
    _link(objs[-1:], CEILING_OUT, verbose)
    return OUT


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
