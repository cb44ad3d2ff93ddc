"""Build libqi.so in-tree for gfx950 with hipcc.

    python -m block_causal_attention_qi_amd.build        # or __graft_entry__.build()

Device code is compiled with packed-fp32 instructions disabled and with floating-point
contraction off (every fused multiply-add in the kernels is written explicitly), and with
correctly rounded float32 division (the fp8 scales a/448 and 448/a are IEEE quotients).
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libqi.so")
SOURCES = ["plan.cpp", "api.hip", "attn_fwd.hip", "prefix_kv.hip"]
ARCH = "gfx950"


def hipcc():
    path = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(path):
        raise RuntimeError("hipcc not found (ROCm is required to build libqi)")
    return path


def flags():
    return ["--offload-arch=" + ARCH, "-O3", "-std=c++17", "-fPIC", "-shared",
            "-ffp-contract=off", "-fhip-fp32-correctly-rounded-divide-sqrt",
            "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
            "-I" + CSRC, "-I" + os.path.join(os.path.dirname(HERE), "include")]


def build_library(verbose=False):
    """Compile every source into libqi.so (always recompiles).  Returns the path."""
    tmp = LIB + ".tmp%d" % os.getpid()
    cmd = [hipcc()] + flags() + [os.path.join(CSRC, s) for s in SOURCES] + ["-o", tmp]
    res = subprocess.run(cmd, capture_output=True, text=True)
    msgs = [l for l in (res.stdout + res.stderr).splitlines() if "packed-fp32-ops" not in l]
    if res.returncode != 0:
        if os.path.exists(tmp):
            os.remove(tmp)
        raise RuntimeError("hipcc failed:\n" + " ".join(cmd) + "\n" + "\n".join(msgs))
    if verbose and msgs:
        print("\n".join(msgs), file=sys.stderr)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build_library(verbose=True))
