"""Build libsla.so (the gfx950 HIP kernels + the C ABI) in-tree with hipcc.

    python -m block_sparse_linear_02_amd.build        # or build() from Python

Every HIP source is compiled for gfx950 only, with packed-fp32 instruction selection switched
off (-Xclang -target-feature -Xclang -packed-fp32-ops), then linked into
block_sparse_linear_02_amd/libsla.so.
"""

from __future__ import annotations

import concurrent.futures
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
OUT = os.path.join(PKG, "libsla.so")
BUILD_DIR = os.path.join(PKG, "_build")

SOURCES = ["router.hip", "linear_state.hip", "linear_gemm.hip", "sparse.hip", "sparse_pair.hip",
           "linear_apply.hip", "fp8.hip", "pisa_stats.hip", "pisa.hip", "branch_drop.hip",
           "bwd.hip", "svoo.hip", "soft.hip", "validate.hip", "api.cpp"]

FLAGS = [
    "-O3",
    "-std=c++17",
    "-fPIC",
    "--offload-arch=gfx950",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-unused-command-line-argument",
    f"-I{INCLUDE}",
    f"-I{CSRC}",
]


def _hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build libsla)")


def _compile(src: str) -> str:
    obj = os.path.join(BUILD_DIR, os.path.basename(src) + ".o")
    lang = ["-x", "hip"] if src.endswith(".cpp") else []
    cmd = [_hipcc(), *FLAGS, *lang, "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"compile failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    return obj


def build(verbose: bool = False) -> str:
    """Compile every source for gfx950 and link libsla.so; returns its path."""
    os.makedirs(BUILD_DIR, exist_ok=True)
    with concurrent.futures.ThreadPoolExecutor(max_workers=min(8, len(SOURCES))) as ex:
        objs = list(ex.map(_compile, SOURCES))
    tmp = OUT + ".tmp"
    cmd = [_hipcc(), "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, OUT)
    if verbose:
        print(f"built {OUT}")
    return OUT


ASAN_DIR = os.path.join(PKG, "_build_asan")
ASAN_OUT = os.path.join(ASAN_DIR, "libsla_asan.so")


def asan_runtime() -> str:
    """The compiler's AddressSanitizer runtime (to preload into a host process using ASAN_OUT)."""
    r = subprocess.run([_hipcc(), "-print-file-name=libclang_rt.asan-x86_64.so"], capture_output=True, text=True)
    path = r.stdout.strip()
    if r.returncode != 0 or not os.path.exists(path):
        raise RuntimeError("the AddressSanitizer runtime of the HIP compiler was not found")
    return path


def build_asan(verbose: bool = False) -> str:
    """A copy of the library with AddressSanitizer on its host code only (argument checks,
    workspace carving, status strings; the device code is built as usual), for CPU tests of
    those paths.  Returns its path."""
    os.makedirs(ASAN_DIR, exist_ok=True)
    flags = [f for f in FLAGS if f != "-O3"] + [
        "-O1", "-g", *"-Xarch_host -fsanitize=address".split(), "-fno-omit-frame-pointer"]

    def comp(src: str) -> str:
        obj = os.path.join(ASAN_DIR, os.path.basename(src) + ".o")
        lang = ["-x", "hip"] if src.endswith(".cpp") else []
        cmd = [_hipcc(), *flags, *lang, "-c", os.path.join(CSRC, src), "-o", obj]
        r = subprocess.run(cmd, capture_output=True, text=True)
        if r.returncode != 0:
            raise RuntimeError(f"compile failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
        return obj

    with concurrent.futures.ThreadPoolExecutor(max_workers=min(8, len(SOURCES))) as ex:
        objs = list(ex.map(comp, SOURCES))
    tmp = ASAN_OUT + ".tmp"
    cmd = [_hipcc(), "--offload-arch=gfx950", "-shared", "-fPIC", *"-Xarch_host -fsanitize=address".split(),
           "-shared-libasan", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, ASAN_OUT)
    if verbose:
        print(f"built {ASAN_OUT}")
    return ASAN_OUT


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
