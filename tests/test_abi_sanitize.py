"""The C ABI's host code under AddressSanitizer and UndefinedBehaviorSanitizer (CPU only).

The ABI translation unit (argument checks, workspace carving, host helpers)
is compiled again with host-only sanitizers (each -fsanitize= behind
-Xarch_host: the device code is built as usual), linked with the other
objects of the normal build into a separate library, and driven by
tests/abi_sanitize/abi_checks.cpp: host helpers at ordinary and extreme
sizes, and every entry point with arguments it rejects before enqueueing
anything.  A sanitizer finding aborts the driver; this test fails on any
non-zero exit.
"""
import glob
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "sparse_mixture_experts_argmax_amd", "csrc")
BUILD = os.path.join(ROOT, "_build")
OUT = os.path.join(BUILD, "sanitize")
CLANG = "/opt/rocm/llvm/bin/clang++"


def _hipcc():
    return shutil.which("hipcc") or "/opt/rocm/bin/hipcc"


@pytest.mark.skipif(not (os.path.exists(_hipcc()) and os.path.exists(CLANG)), reason="no ROCm compilers")
def test_abi_host_code_under_sanitizers():
    objs = [o for o in glob.glob(os.path.join(BUILD, "*.o")) if not o.endswith("moe_api.o")]
    if len(objs) < 5:
        pytest.skip("build the library first (sparse_mixture_experts_argmax_amd/build.py)")
    os.makedirs(OUT, exist_ok=True)
    san = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
           "-Xarch_host", "-fno-sanitize-recover=undefined", "-Xarch_host", "-fno-omit-frame-pointer"]
    api_o = os.path.join(OUT, "moe_api.o")
    subprocess.run([_hipcc(), "--offload-arch=gfx950", "-O1", "-g", "-std=c++17", "-fPIC", "-Xclang",
                    "-target-feature", "-Xclang", "-packed-fp32-ops", *san, "-I", os.path.join(ROOT, "include"),
                    "-I", CSRC, "-c", os.path.join(CSRC, "moe_api.hip"), "-o", api_o],
                   check=True, capture_output=True, timeout=600)
    lib = os.path.join(OUT, "libmoe_san.so")
    subprocess.run([_hipcc(), "--offload-arch=gfx950", "-shared", "-fPIC", api_o, *objs, "-o", lib],
                   check=True, capture_output=True, timeout=600)
    exe = os.path.join(OUT, "abi_checks")
    subprocess.run([CLANG, "-fsanitize=address,undefined", "-fno-sanitize-recover=undefined", "-g", "-O1",
                    "-D__HIP_PLATFORM_AMD__", "-I", os.path.join(ROOT, "include"), "-I", "/opt/rocm/include",
                    os.path.join(ROOT, "tests", "abi_sanitize", "abi_checks.cpp"), lib, f"-Wl,-rpath,{OUT}",
                    "-L/opt/rocm/lib", "-lamdhip64", "-Wl,-rpath,/opt/rocm/lib", "-o", exe],
                   check=True, capture_output=True, timeout=600)
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=1",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1", HIP_VISIBLE_DEVICES="")
    r = subprocess.run([exe], capture_output=True, text=True, timeout=300, env=env)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "abi checks passed" in r.stdout
    assert "runtime error" not in r.stderr and "AddressSanitizer" not in r.stderr, r.stderr
