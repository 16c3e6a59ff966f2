"""Build libq8narrow.so in-tree with hipcc for gfx950.

Flags: -O3, no fast-math, -ffp-contract=off (every fused multiply-add in the
kernels is written out explicitly), and packed-fp32 instructions disabled.
"""

from __future__ import annotations

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB_PATH = os.path.join(HERE, "libq8narrow.so")

SOURCES = ["q8_pack.hip", "q8_matmul.hip", "q8_rope.hip", "q8_measure.hip", "q8_abi.hip",
           "q8_noalloc.hip"]
HEADERS = ["q8_internal.h", "q8_measure.h"]

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"

FLAGS = [
    f"--offload-arch={ARCH}",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-ffp-contract=off",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall",
    "-Wno-unused-function",
    "-I", INCLUDE,
    "-I", CSRC,
]


def build(out: str = LIB_PATH, extra_flags: list[str] | None = None,
          verbose: bool = False) -> str:
    """Compile every source into one shared library at ``out``."""
    srcs = [os.path.join(CSRC, s) for s in SOURCES]
    tmp = out + ".tmp"
    cmd = [HIPCC, *FLAGS, *(extra_flags or []), "-shared", "-o", tmp, *srcs]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    msgs = "\n".join(
        line for line in (res.stdout + res.stderr).splitlines()
        # hipcc's host pass does not know the device-only feature flag
        if "packed-fp32-ops" not in line and "is not a recognized feature" not in line)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed ({res.returncode}):\n{msgs}")
    if verbose and msgs.strip():
        print(msgs, file=sys.stderr)
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    print(build(verbose=True))
