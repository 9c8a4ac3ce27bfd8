"""Build the HIP library ``libringattn.so`` in-tree with hipcc for gfx950."""
from __future__ import annotations

import os
import re
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


# Kernels whose vmcnt waits are counted by hand (wait_vmem<N> in gfx950_tile.h): a spill puts scratch
# loads and stores into the same counter and silently breaks those counts, so the build refuses them.
HAND_COUNTED_WAIT_KERNELS = ("step_mfma_bf16_d128", "bwd_dq_bf16_d128", "bwd_dkv_bf16_d128", "ffn_gemm_bf16")


_REMARK = re.compile(r"remark:(?:\s*\S+:\d+:\d+:)?\s*([A-Za-z][^:\[]*?(?:\[[^\]]*\])?)\s*:\s*(.*?)\s*"
                     r"\[-Rpass-analysis=kernel-resource-usage\]")


def kernel_resources(stderr: str) -> dict:
    """{mangled kernel name: {field: value}} from clang's -Rpass-analysis=kernel-resource-usage remarks."""
    out, cur = {}, None
    for ln in stderr.splitlines():
        mt = _REMARK.search(ln)
        if not mt:
            continue
        key, val = mt.group(1).strip(), mt.group(2).strip()
        if key == "Function Name":
            cur = val
            out[cur] = {}
        elif cur is not None:
            out[cur][key] = val
    return out


def check_no_scratch(resources: dict) -> None:
    """Raise if a kernel with hand-counted memory waits uses scratch memory (VGPR spills or a stack).
    SGPRs spilled into VGPR lanes (v_writelane / v_readlane) issue no memory instructions and pass."""
    bad = []
    for name, fields in resources.items():
        if any(k in name for k in HAND_COUNTED_WAIT_KERNELS):
            scratch = int(fields.get("ScratchSize [bytes/lane]", "0") or 0)
            spills = int(fields.get("VGPRs Spill", "0") or 0)
            if scratch or spills or fields.get("Dynamic Stack", "False") != "False":
                bad.append(f"{name}: scratch {scratch} B/lane, {spills} spilled VGPRs")
    if bad:
        raise RuntimeError("kernels with hand-counted vmcnt waits must not use scratch:\n" + "\n".join(bad))


def hipcc() -> str:
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    return os.path.join(rocm, "bin", "hipcc")


def build(verbose: bool = False) -> str:
    """Compile every HIP source into the shared library next to this file; returns its path."""
    srcs = [os.path.join(CSRC, s) for s in SOURCES]
    tmp = LIB_PATH + ".tmp"
    cmd = [hipcc(), *HIPCC_FLAGS, "-Rpass-analysis=kernel-resource-usage", "-I", INCLUDE, "-I", CSRC, *srcs,
           "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    # hipcc's host pass does not know the packed-fp32 target feature and says so; that is harmless
    noise = [ln for ln in res.stderr.splitlines()
             if "packed-fp32-ops" not in ln and "kernel-resource-usage" not in ln and ln.strip()]
    if res.returncode != 0:
        raise RuntimeError("hipcc failed:\n" + "\n".join(noise))
    if verbose and noise:
        print("\n".join(noise), file=sys.stderr)
    resources = kernel_resources(res.stderr)
    if not any(any(k in n for k in HAND_COUNTED_WAIT_KERNELS) for n in resources):
        raise RuntimeError("hipcc printed no resource-usage remarks for the MFMA kernels")
    try:
        check_no_scratch(resources)
    except RuntimeError:
        os.remove(tmp)
        raise
    os.replace(tmp, LIB_PATH)
    return LIB_PATH


if __name__ == "__main__":
    print(build(verbose=True))
