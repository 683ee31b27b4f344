"""Build the HIP library of the MoE layer for gfx950 (MI355X), in-tree.

    python -m mixture_experts_layer_sort_amd.build

compiles every ``csrc/*.hip`` kernel source and ``csrc/api.cpp`` with hipcc
into ``libmoe_mi355x.so`` next to this file.  Packed-FP32 instructions are
disabled for the device code (``-packed-fp32-ops``).
"""
from __future__ import annotations

import glob
import os
import subprocess
import sys

PKG_DIR = os.path.dirname(os.path.abspath(__file__))
REPO_DIR = os.path.dirname(PKG_DIR)
CSRC = os.path.join(PKG_DIR, "csrc")
INCLUDE = os.path.join(REPO_DIR, "include")
LIB_NAME = "libmoe_mi355x.so"
LIB_PATH = os.path.join(PKG_DIR, LIB_NAME)
ARCH = "gfx950"


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", "hipcc"):
        if cand and (os.path.isabs(cand) and os.path.exists(cand) or not os.path.isabs(cand)):
            return cand
    return "hipcc"


def sources() -> list:
    return sorted(glob.glob(os.path.join(CSRC, "*.hip"))) + [os.path.join(CSRC, "api.cpp")]


def build(verbose: bool = False, extra_flags=None) -> str:
    """Compile the library; returns its path.  Raises CalledProcessError on failure."""
    out_tmp = LIB_PATH + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-shared",
           "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
           "-Wno-unused-command-line-argument",
           f"-I{INCLUDE}", f"-I{CSRC}", "-o", out_tmp]
    cmd += list(extra_flags or [])
    # api.cpp is host C++ that includes HIP headers; compile every file as HIP
    srcs = sources()
    cmd += ["-x", "hip"] + srcs
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    out = "\n".join(l for l in res.stdout.splitlines() if "packed-fp32-ops" not in l)
    if res.returncode != 0:
        sys.stderr.write(out + "\n")
        raise subprocess.CalledProcessError(res.returncode, cmd, output=out)
    if verbose and out.strip():
        print(out)
    os.replace(out_tmp, LIB_PATH)
    return LIB_PATH


if __name__ == "__main__":
    print(build(verbose=True))
