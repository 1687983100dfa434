"""The host layer under AddressSanitizer and UndefinedBehaviorSanitizer (CPU).

ts_api.cpp (argument checks, planning, workspace carving, launch sequencing)
is compiled with host-side sanitizers, linked against stand-in launchers
that enqueue nothing (tests/host_sanitize/stub_launchers.cpp), and driven
through the whole C ABI by tests/host_sanitize/abi_driver.cpp: about two
million calls over a grid of layouts, batch sizes and k, valid, invalid and
extreme (int32 limits). The device code of ts_api.cpp is built without
sanitizers. Any sanitizer report aborts the driver; the test wants exit 0.
"""
import os
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
OUT = os.path.join(ROOT, "sparse_kv_cache_ts_amd", "_build", "san")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
CLANG = "/opt/rocm/llvm/bin/clang++"

# host-side sanitizers only: each -fsanitize follows -Xarch_host on the hipcc line
HIP_FLAGS = ["-std=c++17", "-O1", "-g", "--offload-arch=gfx950",
             "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
             "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
             "-Xarch_host", "-fno-sanitize-recover=all", "-Xarch_host", "-fno-omit-frame-pointer",
             "-I", os.path.join(ROOT, "include"), "-I", os.path.join(ROOT, "sparse_kv_cache_ts_amd", "csrc")]
HOST_SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer"]


def _run(cmd):
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, f"{' '.join(cmd)}\n{r.stdout[-4000:]}\n{r.stderr[-4000:]}"


@pytest.mark.skipif(not (os.path.exists(HIPCC) and os.path.exists(CLANG)), reason="needs hipcc and clang++")
def test_host_layer_under_asan_and_ubsan():
    os.makedirs(OUT, exist_ok=True)
    objs = []
    for src, name in ((os.path.join(ROOT, "sparse_kv_cache_ts_amd", "csrc", "ts_api.cpp"), "ts_api.o"),
                      (os.path.join(ROOT, "tests", "host_sanitize", "stub_launchers.cpp"), "stubs.o")):
        objs.append(os.path.join(OUT, name))
        _run([HIPCC, "-x", "hip", *HIP_FLAGS, "-c", src, "-o", objs[-1]])
    objs.append(os.path.join(OUT, "driver.o"))
    _run([CLANG, "-std=c++17", "-O1", "-g", *HOST_SAN, "-I", os.path.join(ROOT, "include"),
          "-c", os.path.join(ROOT, "tests", "host_sanitize", "abi_driver.cpp"), "-o", objs[-1]])
    exe = os.path.join(OUT, "abi_driver")
    _run([CLANG, *HOST_SAN, *objs, "-L/opt/rocm/lib", "-lamdhip64", "-Wl,-rpath,/opt/rocm/lib", "-o", exe])
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=0",
               UBSAN_OPTIONS="print_stacktrace=1")
    r = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=600)
    out = r.stdout + r.stderr
    assert "runtime error" not in out and "AddressSanitizer" not in out, out[-6000:]
    assert r.returncode == 0, out[-6000:]
    assert " 0 failed" in r.stdout, r.stdout[-3000:]
