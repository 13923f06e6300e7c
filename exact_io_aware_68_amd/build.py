"""Build libfa.so (the C-ABI attention library) for gfx950 with hipcc, in-tree.

    python -m exact_io_aware_68_amd.build [--verbose]

Each .hip file under csrc/ is compiled to an object in parallel, then linked into
exact_io_aware_68_amd/libfa.so.  No JIT cache is involved: the built library sits next to this
file, so it travels with the source tree.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
OUT = os.path.join(PKG, "libfa.so")
BUILD_DIR = os.path.join(PKG, "_build")
ARCH = "gfx950"

# -packed-fp32-ops: keep the compiler from forming packed fp32 VALU ops (v_pk_*_f32).
DEVICE_FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-I", INCLUDE, "-I", CSRC,
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-unused-command-line-argument",
]


# Per-source extra flags.  Every bf16 kernel keeps its MFMA results in ordinary VGPRs: the score
# tiles are post-processed by VALU code every step.  Left to its heuristics the compiler picks
# accumulation registers for all MFMAs of a kernel that needs more than 256 registers (dK/dV),
# and then copies the score tiles out and the long-lived dK, dV accumulators in and out of them
# on every iteration (about 240 copies per 64 MFMAs); with this flag it spills a few loop-
# invariant values to accumulation registers instead.
FILE_FLAGS = {
    "fa_fwd_bf16.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"],
    "fa_bwd_dq.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"],
    "fa_bwd_bf16.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"],
}


def _hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build the attention library)")


def _compile(src: str, verbose: bool) -> str:
    obj = os.path.join(BUILD_DIR, os.path.basename(src) + ".o")
    cmd = [_hipcc(), "-c", src, "-o", obj, *DEVICE_FLAGS,
           *FILE_FLAGS.get(os.path.basename(src), [])]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{r.stdout}\n{r.stderr}")
    return obj


def build(verbose: bool = False) -> str:
    """Compile every kernel source and link libfa.so; returns its path."""
    os.makedirs(BUILD_DIR, exist_ok=True)
    srcs = sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC) if f.endswith(".hip"))
    with cf.ThreadPoolExecutor(max_workers=min(8, len(srcs))) as ex:
        objs = list(ex.map(lambda s: _compile(s, verbose), srcs))
    tmp = OUT + ".tmp"
    cmd = [_hipcc(), "-shared", "-fPIC", f"--offload-arch={ARCH}", *objs, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, OUT)
    return OUT


if __name__ == "__main__":
    print(build(verbose="--verbose" in sys.argv))
