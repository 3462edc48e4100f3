"""Build the C ABI round-trip program (tests/c_abi/ce_roundtrip.cpp) in-tree:
plain host C++ compiled with g++ against the in-tree liblmhead.so and the HIP
runtime, with no Python or torch between the program and the library."""

from __future__ import annotations

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
SRC = os.path.join(HERE, "ce_roundtrip.cpp")
PROG = os.path.join(HERE, "ce_roundtrip")


def build() -> str:
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    pkg = os.path.join(ROOT, "chunked_lm_head_amd")
    cmd = ["g++", "-O2", "-std=c++17", "-Wall", "-D__HIP_PLATFORM_AMD__",
           "-I", os.path.join(ROOT, "include"), "-I", os.path.join(rocm, "include"), SRC,
           "-L", pkg, "-llmhead", "-L", os.path.join(rocm, "lib"), "-lamdhip64",
           "-Wl,-rpath,$ORIGIN/../../chunked_lm_head_amd", "-Wl,-rpath," + os.path.join(rocm, "lib"),
           "-o", PROG + ".tmp"]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        sys.stderr.write(res.stdout + res.stderr)
        raise RuntimeError("g++ failed to build the C ABI round-trip program")
    os.replace(PROG + ".tmp", PROG)
    return PROG


if __name__ == "__main__":
    print(build())
