"""Build the gfx950 shared library ``libmla_verify.so`` in-tree with hipcc.

Run as ``python -m speculative_verify_attention_absorbed_amd._build`` or call
``build()``.  It always recompiles.
"""
from __future__ import annotations

import os
import subprocess
import sys

PKG_DIR = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG_DIR)
CSRC = os.path.join(PKG_DIR, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB_NAME = "libmla_verify.so"
LIB_PATH = os.path.join(PKG_DIR, LIB_NAME)
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

SOURCES = ["mla_verify_kernels.hip", "mla_kv_update.hip", "mla_verify_host.cpp"]

# -packed-fp32-ops: keep the compiler from emitting packed fp32 VALU ops
# (v_pk_fma_f32 and friends); it is a device-side feature flag.
# kernarg preload: the leading 10 kernel arguments arrive in SGPRs at wave
# start instead of through a scalar memory round trip.
DEVICE_FLAGS = ["--offload-arch=gfx950", "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
                "-mllvm", "-amdgpu-kernarg-preload-count=10"]
COMMON_FLAGS = ["-O3", "-std=c++17", "-fPIC", "-Wall", "-Wno-unused-function"]


def build(verbose: bool = False) -> str:
    """Compile every source and link ``libmla_verify.so``; returns its path."""
    tmp = LIB_PATH + ".tmp"
    cmd = [HIPCC, *DEVICE_FLAGS, *COMMON_FLAGS, "-shared", "-I", INCLUDE, "-I", CSRC,
           *[os.path.join(CSRC, s) for s in SOURCES], "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    proc = subprocess.run(cmd, capture_output=True, text=True)
    noise = "is not a recognized feature for this target"
    msgs = "\n".join(line for line in (proc.stdout + proc.stderr).splitlines() if noise not in line)
    if proc.returncode != 0:
        raise RuntimeError(f"hipcc failed ({proc.returncode}):\n{msgs}")
    if verbose and msgs.strip():
        print(msgs)
    os.replace(tmp, LIB_PATH)
    return LIB_PATH


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
