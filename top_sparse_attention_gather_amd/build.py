"""Build the gfx950 shared library in-tree with hipcc.

    python -m top_sparse_attention_gather_amd.build

produces top_sparse_attention_gather_amd/_lib/libsparse_attn.so from the
HIP sources under csrc/ (kernels + the C ABI declared in
include/sparse_attn.h).  Always recompiles.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
LIBDIR = os.path.join(PKG, "_lib")
LIB = os.path.join(LIBDIR, "libsparse_attn.so")

SOURCES = ["sa_api.hip", "sa_bwd_rows.hip", "sa_bwd_mla.hip", "sa_bwd_blk.hip", "sa_fwd_rows.hip", "sa_csr.hip",
           "sa_reduce.hip", "sa_indexer.hip", "sa_noalloc.hip"]

HIPCC_FLAGS = [
    "--offload-arch=gfx950",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-shared",
    # hipcc emits packed fp32 ops on its own from ordinary float code; keep
    # them off (some of their forms have misbehaved on these parts).
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-unused-variable",
    "-Wno-unused-parameter",
]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm toolchain required to build the library)")


def build(verbose: bool = False) -> str:
    os.makedirs(LIBDIR, exist_ok=True)
    srcs = [os.path.join(CSRC, s) for s in SOURCES]
    tmp = LIB + ".tmp"
    cmd = [hipcc(), *HIPCC_FLAGS, "-I", os.path.join(ROOT, "include"), "-I", CSRC, *srcs, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed ({r.returncode}):\n{r.stdout}\n{r.stderr}")
    # hipcc's host pass does not know the packed-fp32 target feature and
    # warns about it; anything else is worth showing.
    noise = [ln for ln in r.stderr.splitlines() if ln.strip() and "packed-fp32-ops" not in ln]
    if verbose and noise:
        print("\n".join(noise), file=sys.stderr)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
