"""In-tree build of ``libqmoe.so`` for gfx950 with hipcc (no JIT, no torch extension).

``python -m quantized_moe_expert_topk_amd.build`` compiles every source in ``csrc/`` to an
object (in parallel) and links the shared library next to this file.
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
LIB_PATH = os.path.join(PKG, "libqmoe.so")
BUILD_DIR = os.path.join(PKG, "_build")

ARCH = "gfx950"
# -packed-fp32-ops: keep the compiler from forming packed fp32 VALU instructions.
HIPCC_FLAGS = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}", "-Xclang", "-target-feature",
               "-Xclang", "-packed-fp32-ops", "-I", INCLUDE, "-I", CSRC, "-Wall", "-Wno-unused-function"]
# Per-file options.  The MXFP4 streaming kernels measured faster with the backend's
# memory-clause scheduler, which groups their weight loads into longer clauses; the same option
# slowed the other formats' kernels, so it is given to the file that instantiates MXFP4 only.
FILE_FLAGS = {"expert_mxfp4.hip": ["-mllvm", "-amdgpu-sched-strategy=max-memory-clause"]}


def _hipcc() -> str:
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if c and os.path.exists(c):
            return c
    raise RuntimeError("hipcc not found (ROCm is required to build libqmoe.so)")


def sources():
    return sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC) if f.endswith((".hip", ".cpp")))


def build(verbose: bool = False) -> str:
    """Compile all sources and link ``libqmoe.so``; always rebuilds."""
    hipcc = _hipcc()
    os.makedirs(BUILD_DIR, exist_ok=True)
    srcs = sources()

    def compile_one(src):
        obj = os.path.join(BUILD_DIR, os.path.basename(src) + ".o")
        lang = ["-x", "hip"] if src.endswith(".hip") else []
        cmd = [hipcc, *HIPCC_FLAGS, *FILE_FLAGS.get(os.path.basename(src), []), *lang, "-c", src, "-o", obj]
        r = subprocess.run(cmd, capture_output=True, text=True)
        out = "\n".join(l for l in (r.stdout + r.stderr).splitlines()
                        if "packed-fp32-ops' is not a recognized feature" not in l)
        if r.returncode != 0:
            raise RuntimeError(f"compile failed: {' '.join(cmd)}\n{out}")
        if verbose and out.strip():
            print(out, file=sys.stderr)
        return obj

    with ThreadPoolExecutor(max_workers=min(8, len(srcs))) as ex:
        objs = list(ex.map(compile_one, srcs))
    tmp = LIB_PATH + ".tmp"
    # --no-undefined: a missing definition fails here, not when the library is loaded
    cmd = [hipcc, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-Wl,--no-undefined", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed: {' '.join(cmd)}\n{r.stdout}{r.stderr}")
    os.replace(tmp, LIB_PATH)
    return LIB_PATH


if __name__ == "__main__":
    print(build(verbose=True))
