"""Build libmoe.so (the HIP kernels and the C ABI) for gfx950 with hipcc.

Every .hip file under csrc/ is compiled to an object in _build/ (in
parallel), then linked into sparse_mixture_experts_argmax_amd/libmoe.so.
Run: python sparse_mixture_experts_argmax_amd/build.py [--incremental]  (by path:
importing the package loads the library this script builds)
"""
from __future__ import annotations

import glob
import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD_DIR = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libmoe.so")
ARCH = os.environ.get("MOE_OFFLOAD_ARCH", "gfx950")

FLAGS = [
    f"--offload-arch={ARCH}",
    "-O3",
    "-std=c++17",
    "-fPIC",
    # keep hipcc from forming packed fp32 ops (v_pk_*_f32) on its own
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", INCLUDE,
    "-I", CSRC,
]


def hipcc() -> str:
    p = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(p):
        raise RuntimeError("hipcc not found; the HIP library cannot be built")
    return p


def _compile(src: str, obj: str) -> None:
    cmd = [hipcc(), *FLAGS, "-c", src, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{r.stderr}")
    # the host pass of hipcc does not know the gpu-only feature flag; drop that note
    noise = "'-packed-fp32-ops' is not a recognized feature"
    for line in r.stderr.splitlines():
        if line.strip() and noise not in line:
            print(line, file=sys.stderr)


def _stale(src: str, obj: str, headers: list) -> bool:
    """An object older than its source or than any header (sources include several)."""
    if not os.path.exists(obj):
        return True
    t = os.path.getmtime(obj)
    return any(os.path.getmtime(p) > t for p in [src, *headers])


def _digest_object() -> str:
    """moe_source_digest(): the digest of the sources being built, in an object
    of its own (source_digest.py by path, like this script)."""
    import importlib.util
    spec = importlib.util.spec_from_file_location("_moe_digest", os.path.join(PKG, "source_digest.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    src = os.path.join(BUILD_DIR, "source_digest.cpp")
    obj = os.path.join(BUILD_DIR, "source_digest.o")
    with open(src, "w") as fh:
        fh.write("// written by build.py: the digest of the sources this library is built from\n"
                 f'extern "C" const char *moe_source_digest(void) {{ return "{mod.source_digest(CSRC)}"; }}\n')
    r = subprocess.run(["g++", "-O2", "-fPIC", "-c", src, "-o", obj], capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"g++ failed on {src}:\n{r.stderr}")
    return obj


def build(jobs: int | None = None, incremental: bool = False) -> str:
    """Compile every .hip file and link libmoe.so.  incremental=True recompiles
    only the objects that are older than their source or any header."""
    os.makedirs(BUILD_DIR, exist_ok=True)
    srcs = sorted(glob.glob(os.path.join(CSRC, "*.hip")))
    objs = [os.path.join(BUILD_DIR, os.path.basename(s)[:-4] + ".o") for s in srcs]
    headers = sorted(glob.glob(os.path.join(CSRC, "*.h")) + glob.glob(os.path.join(INCLUDE, "*.h")))
    todo = [(s, o) for s, o in zip(srcs, objs) if not incremental or _stale(s, o, headers)]
    n = jobs or min(8, max(1, len(todo)), os.cpu_count() or 1)
    with ThreadPoolExecutor(n) as ex:
        list(ex.map(lambda so: _compile(*so), todo))
    objs = objs + [_digest_object()]
    tmp = LIB + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr}")
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(incremental="--incremental" in sys.argv[1:]))
