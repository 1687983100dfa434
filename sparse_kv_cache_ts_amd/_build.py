"""Build libts.so (HIP kernels + C ABI) for gfx950 with hipcc.

Usage: python -m sparse_kv_cache_ts_amd._build   (or call build()).
Objects go to sparse_kv_cache_ts_amd/_build/, the library to
sparse_kv_cache_ts_amd/libts.so. Every call recompiles.
"""
from __future__ import annotations

import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
OUT_DIR = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libts.so")
ARCH = os.environ.get("TS_OFFLOAD_ARCH", "gfx950")

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
COMMON = [
    "-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
    # no packed fp32 instructions anywhere in the device code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", os.path.join(ROOT, "include"), "-I", CSRC,
    "-Wall", "-Wno-unused-function",
]


def sources() -> list:
    names = sorted(f for f in os.listdir(CSRC) if f.endswith(".hip") or f.endswith(".cpp"))
    return [os.path.join(CSRC, f) for f in names]


def _compile(src: str, out_dir: str = OUT_DIR) -> str:
    obj = os.path.join(out_dir, os.path.basename(src) + ".o")
    cmd = [HIPCC, *COMMON, "-x", "hip", "-c", src, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{r.stderr}")
    return obj


def build(verbose: bool = True) -> str:
    """Compile every source and link the in-tree libts.so."""
    out_dir, lib = OUT_DIR, LIB
    os.makedirs(out_dir, exist_ok=True)
    srcs = sources()
    jobs = min(len(srcs), int(os.environ.get("MAX_JOBS", "8")), 16)
    with ThreadPoolExecutor(max_workers=max(1, jobs)) as ex:
        objs = list(ex.map(lambda f: _compile(f, out_dir), srcs))
    tmp = lib + ".tmp"
    cmd = [HIPCC, "-shared", "-fPIC", f"--offload-arch={ARCH}", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr}")
    os.replace(tmp, lib)
    if verbose:
        print(f"built {lib} from {len(srcs)} sources for {ARCH}")
    return lib


if __name__ == "__main__":
    build()
    sys.exit(0)
