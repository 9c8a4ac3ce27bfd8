"""Build the HIP library ``libringattn.so`` in-tree with hipcc for gfx950."""
from __future__ import annotations

import os
import subprocess
import sys

PKG_DIR = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG_DIR)
CSRC = os.path.join(PKG_DIR, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB_NAME = "libringattn.so"
LIB_PATH = os.path.join(PKG_DIR, LIB_NAME)

SOURCES = ["api.hip", "step_mfma_bf16.hip", "step_generic.hip", "bwd_mfma_bf16.hip", "bwd_generic.hip",
           "ffn_mfma_bf16.hip"]

HIPCC_FLAGS = [
    "--offload-arch=gfx950",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-shared",
    "-Wall",
    "-Wno-unused-result",
    # packed fp32 VALU forms stay off (compiler-generated v_pk_*_f32 are not used)
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
]


def hipcc() -> str:
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    return os.path.join(rocm, "bin", "hipcc")


def build(verbose: bool = False) -> str:
    """Compile every HIP source into the shared library next to this file; returns its path."""
    srcs = [os.path.join(CSRC, s) for s in SOURCES]
    tmp = LIB_PATH + ".tmp"
    cmd = [hipcc(), *HIPCC_FLAGS, "-I", INCLUDE, "-I", CSRC, *srcs, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    # hipcc's host pass does not know the packed-fp32 target feature and says so; that is harmless
    noise = [ln for ln in res.stderr.splitlines() if "packed-fp32-ops" not in ln and ln.strip()]
    if res.returncode != 0:
        raise RuntimeError("hipcc failed:\n" + "\n".join(noise))
    if verbose and noise:
        print("\n".join(noise), file=sys.stderr)
    os.replace(tmp, LIB_PATH)
    return LIB_PATH


if __name__ == "__main__":
    print(build(verbose=True))
