"""Build the HIP library libcsa.so for gfx950, in-tree.

    python -m compressed_attention_long_amd.build

compiles every csrc/*.hip (objects under _build/) and links
compressed_attention_long_amd/libcsa.so with hipcc.
"""
from __future__ import annotations

import glob
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
LIB = os.path.join(PKG, "libcsa.so")
ARCH = "gfx950"

HIPCC_FLAGS = [
    f"--offload-arch={ARCH}",
    "-O3",
    "-std=c++17",
    "-fPIC",
    # packed fp32 instructions are kept out of every kernel
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-unused-command-line-argument",
]
# MFMA accumulators in VGPRs: avoids AGPR<->VGPR copies around the softmax / ReLU epilogues.
PER_FILE_FLAGS = {
    "attend.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"],
    "indexer.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"],
    "compress.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"],
}
BUILD_DIR = os.path.join(ROOT, "_build")


def hipcc() -> str:
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if c and os.path.exists(c):
            return c
    raise RuntimeError("hipcc not found: the CSA library needs ROCm's hipcc to build")


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    return subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)


def _check(proc, what, verbose):
    out, _ = proc.communicate()
    msgs = "\n".join(l for l in out.splitlines() if "packed-fp32-ops" not in l and l.strip())
    if proc.returncode != 0:
        raise RuntimeError(f"hipcc failed on {what} ({proc.returncode}):\n{msgs}")
    if verbose and msgs:
        print(msgs, flush=True)


def build(verbose: bool = False, extra_flags=()) -> str:
    """Compile csrc/*.hip (in parallel, one object each) and link libcsa.so (always recompiles)."""
    srcs = sorted(glob.glob(os.path.join(CSRC, "*.hip")))
    os.makedirs(BUILD_DIR, exist_ok=True)
    inc = ["-I", os.path.join(ROOT, "include")]
    objs, procs = [], []
    for src in srcs:
        obj = os.path.join(BUILD_DIR, os.path.basename(src) + ".o")
        flags = [*HIPCC_FLAGS, *PER_FILE_FLAGS.get(os.path.basename(src), []), *extra_flags]
        procs.append((_run([hipcc(), *flags, *inc, "-c", src, "-o", obj], verbose), src))
        objs.append(obj)
    for proc, src in procs:
        _check(proc, os.path.basename(src), verbose)
    tmp = LIB + ".tmp"
    _check(_run([hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp], verbose), "link", verbose)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
