"""Compile libpkv.so (host library + gfx950 kernels) in-tree with hipcc.

Every source is compiled to an object in parallel (the kernel units take
most of the time), then the objects are linked into libpkv.so."""
from __future__ import annotations

import os
import subprocess
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libpkv.so")
SOURCES = [os.path.join(CSRC, n) for n in
           ("pool.cpp", "sched.cpp", "plan.cpp", "append.hip", "decode.hip", "prefill.hip")]

# -packed-fp32-ops: keep the compiler from emitting packed fp32 VALU forms.
HIPCC_FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-unused-result",
]


def build(verbose: bool = False, extra_flags=(), out: str | None = None) -> str:
    """Build libpkv.so (or `out`), with extra compiler flags if given."""
    hipcc = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
    out = out or LIB
    objdir = os.path.join(os.path.dirname(out), "_build")
    os.makedirs(objdir, exist_ok=True)
    inc = ["-I", os.path.join(HERE, "..", "include")]

    def compile_one(src):
        obj = os.path.join(objdir, os.path.basename(src) + ".o")
        r = subprocess.run([hipcc, *HIPCC_FLAGS, *extra_flags, *inc, "-c", src, "-o", obj],
                           capture_output=True, text=True)
        if r.returncode != 0:
            raise RuntimeError(f"hipcc failed on {os.path.basename(src)} ({r.returncode}):\n{r.stderr}")
        if verbose and r.stderr:
            print(r.stderr)
        return obj

    with ThreadPoolExecutor(max_workers=len(SOURCES)) as ex:
        objs = list(ex.map(compile_one, SOURCES))
    tmp = out + ".tmp"
    r = subprocess.run([hipcc, "--offload-arch=gfx950", "-shared", "-fPIC", *objs, "-o", tmp],
                       capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed ({r.returncode}):\n{r.stderr}")
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    print(build(verbose=True))
