"""Build libec.so (the HIP kernels and the C ABI) in-tree for gfx950.

    python -m entropy_guided_kv_amd.build

Each .hip file under csrc/ is compiled with hipcc to an object in _build/ and
the objects are linked into entropy_guided_kv_amd/libec.so. Compiles every
time it is called (sources are few; a full build takes well under a minute
with parallel jobs).
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libec.so")
ARCH = "gfx950"


def hipcc() -> str:
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if c and os.path.exists(c):
            return c
    raise RuntimeError("hipcc not found (ROCm is required to build libec.so)")


def sources():
    return sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC) if f.endswith(".hip"))


def common_flags(debug: bool = False):
    flags = [
        f"--offload-arch={ARCH}",
        "-std=c++17",
        "-fPIC",
        "-O3" if not debug else "-O1",
        # no packed-fp32 instructions in generated code
        "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
        "-I", INCLUDE,
        "-I", CSRC,
        "-Wno-unused-result",
    ]
    if debug:
        flags += ["-g"]
    return flags


def build(verbose: bool = False, jobs: int = 0, debug: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    cc = hipcc()
    srcs = sources()
    objs = [os.path.join(BUILD, os.path.basename(s)[:-4] + ".o") for s in srcs]
    flags = common_flags(debug)

    def compile_one(pair):
        src, obj = pair
        cmd = [cc, *flags, "-c", src, "-o", obj]
        if verbose:
            print(" ".join(cmd), flush=True)
        r = subprocess.run(cmd, capture_output=True, text=True)
        if r.returncode != 0:
            raise RuntimeError(f"hipcc failed for {os.path.basename(src)}:\n{r.stderr[-6000:]}")
        return r.stderr

    jobs = jobs or min(8, os.cpu_count() or 1, len(srcs))
    with ThreadPoolExecutor(jobs) as ex:
        list(ex.map(compile_one, zip(srcs, objs)))
    tmp = LIB + ".tmp"
    # -z defs: every symbol the library references must resolve at link time (a kernel
    # whose host stub the compiler dropped would otherwise surface only at load time)
    cmd = [cc, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-Wl,-z,defs", "-o", tmp, *objs]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr[-6000:]}")
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv, debug="--debug" in sys.argv))
