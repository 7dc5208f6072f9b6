"""Build libjattn.so in-tree for gfx950 with hipcc (no JIT cache, no torch extension machinery).

    python -m diffusion_transformer_joint_amd.build [--verbose]
"""
from __future__ import annotations

import concurrent.futures
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD_DIR = os.path.join(ROOT, "_build")
LIB_PATH = os.path.join(PKG, "libjattn.so")

SOURCES = ["jattn_prenorm.hip", "jattn_fwd.hip", "jattn_bwd.hip", "jattn_bwd_wide.hip", "jattn_api.cpp",
           "adaln_qkv.hip", "adaln_api.cpp", "mlp_api.cpp", "jattn_diag.hip"]
ARCH = "gfx950"

# Packed fp32 VALU instructions are kept out of the code objects (the backend would otherwise form
# them from plain float code); the host pass does not know the feature and warns, harmlessly.
DEVICE_FLAGS = ["-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]
# The attention kernels keep their MFMA accumulators in VGPRs: the score tiles feed VALU work right
# away, and the AGPR form costs two copies per element plus a hazard wait. The projection GEMMs hold
# 256 accumulators per lane and need the AGPRs, and so do the backward kernels of head dims above 72
# (one wave per SIMD, 128 dK/dV accumulator floats per lane at D = 128).
VGPR_ACC = ["-mllvm", "-amdgpu-mfma-vgpr-form"]
AGPR_ACC_SOURCES = {"adaln_qkv.hip", "jattn_bwd_wide.hip"}
COMMON_FLAGS = ["-O3", "-std=c++17", "-fPIC", "-Wall", "-Wno-unused-function",
                f"-I{INCLUDE}", f"-I{CSRC}"]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm toolchain required to build libjattn.so)")


def _compile(src: str, verbose: bool) -> str:
    obj = os.path.join(BUILD_DIR, os.path.basename(src) + ".o")
    cmd = [hipcc(), f"--offload-arch={ARCH}", *COMMON_FLAGS, *DEVICE_FLAGS]
    if src not in AGPR_ACC_SOURCES:
        cmd += VGPR_ACC
    if src.endswith(".cpp"):
        cmd += ["-x", "hip"]
    cmd += ["-c", os.path.join(CSRC, src), "-o", obj]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    noise = "is not a recognized feature for this target"
    err = "\n".join(l for l in r.stderr.splitlines() if noise not in l)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{err}")
    if verbose and err.strip():
        print(err, flush=True)
    return obj


def build(verbose: bool = False) -> str:
    """Compile every source for gfx950 and link libjattn.so next to this file. Always rebuilds."""
    os.makedirs(BUILD_DIR, exist_ok=True)
    with concurrent.futures.ThreadPoolExecutor(max_workers=len(SOURCES)) as ex:
        objs = list(ex.map(lambda s: _compile(s, verbose), SOURCES))
    tmp = LIB_PATH + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr}")
    os.replace(tmp, LIB_PATH)
    return LIB_PATH


if __name__ == "__main__":
    print(build(verbose="--verbose" in sys.argv))
