"""Build libq8narrow.so, and its timeline build libq8narrow_timeline.so,
in-tree with hipcc for gfx950.

Flags: -O3, no fast-math, -ffp-contract=off (every fused multiply-add in the
kernels is written out explicitly), and packed-fp32 instructions disabled.
The timeline build adds -DQ8_TIMELINE (per-wave real-time counter records,
include/q8timeline.h); nothing else differs.
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
TIMELINE_LIB_PATH = os.path.join(HERE, "libq8narrow_timeline.so")

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


def _filtered(text: str) -> str:
    return "\n".join(
        line for line in text.splitlines()
        # hipcc's host pass does not know the device-only feature flag
        if "packed-fp32-ops" not in line and "is not a recognized feature" not in line)


def _start(out: str, extra_flags: list[str], verbose: bool) -> tuple:
    srcs = [os.path.join(CSRC, s) for s in SOURCES]
    tmp = out + ".tmp"
    cmd = [HIPCC, *FLAGS, *extra_flags, "-shared", "-o", tmp, *srcs]
    if verbose:
        print(" ".join(cmd), flush=True)
    proc = subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    return proc, tmp, out


def _finish(job: tuple, verbose: bool) -> str:
    proc, tmp, out = job
    text, _ = proc.communicate()
    msgs = _filtered(text)
    if proc.returncode != 0:
        raise RuntimeError(f"hipcc failed ({proc.returncode}) building {out}:\n{msgs}")
    if verbose and msgs.strip():
        print(msgs, file=sys.stderr)
    os.replace(tmp, out)
    return out


def build(out: str = LIB_PATH, extra_flags: list[str] | None = None,
          verbose: bool = False) -> str:
    """Compile every source into one shared library at ``out``."""
    return _finish(_start(out, list(extra_flags or []), verbose), verbose)


def build_all(verbose: bool = False) -> list[str]:
    """The product library and its timeline build, compiled side by side."""
    jobs = [_start(LIB_PATH, [], verbose),
            _start(TIMELINE_LIB_PATH, ["-DQ8_TIMELINE"], verbose)]
    return [_finish(j, verbose) for j in jobs]


if __name__ == "__main__":
    print("\n".join(build_all(verbose=True)))
