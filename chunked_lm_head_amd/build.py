"""Build liblmhead.so (HIP, gfx950) in-tree with hipcc."""

from __future__ import annotations

import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "liblmhead.so")
SOURCES = ["lmhead_kernels.hip", "lmhead_candidates.hip", "lmhead_api.hip"]
HEADERS = ["gemm_core.h", "lmhead_kernels.h"]

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = [
    "--offload-arch=gfx950",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-shared",
    # packed fp32 VALU ops (v_pk_*_f32) stay off everywhere in this library
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-unused-command-line-argument",
]


def sources():
    return [os.path.join(CSRC, s) for s in SOURCES]


def build(verbose: bool = False, extra_flags=None) -> str:
    cmd = [HIPCC, *FLAGS, *(extra_flags or []), "-I", INCLUDE, "-I", CSRC, *sources(), "-o", LIB + ".tmp"]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        sys.stderr.write(res.stdout + res.stderr)
        raise RuntimeError("hipcc failed to build liblmhead.so")
    # hipcc's host pass does not know the packed-fp32 feature; that warning is expected
    noise = "'-packed-fp32-ops' is not a recognized feature"
    rest = [ln for ln in (res.stdout + res.stderr).splitlines() if noise not in ln and ln.strip()]
    if rest and verbose:
        sys.stderr.write("\n".join(rest) + "\n")
    os.replace(LIB + ".tmp", LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
