"""Build the gfx950 attention library in place: exact_attention_prefill_amd/libattn.so.

    python -m exact_attention_prefill_amd.build

Compiles every kernel instance with hipcc for gfx950 only.  Packed fp32 vector
instructions are switched off on purpose (-packed-fp32-ops): the compiler is free
to form them from scalar float code otherwise.  NaN inputs are outside the
library's contract, so IEEE NaN quieting is off (-fno-honor-nans,
-mno-amdgpu-ieee); infinities keep their meaning.
"""

from __future__ import annotations

import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
LIB = os.path.join(PKG, "libattn.so")
SOURCES = ["attn_api.hip", "prefill.hip", "decode.hip", "bwd.hip"]
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

FLAGS = [
    "--offload-arch=gfx950",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-shared",
    "-Wall",
    "-Wno-unused-function",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # Inputs are finite by contract (infinities are used internally for masking, NaNs
    # never): without IEEE NaN quieting, fmax chains become v_max3 with no
    # canonicalising moves in front of every operand.
    "-fno-honor-nans",
    "-mno-amdgpu-ieee",
    "-I", os.path.join(ROOT, "include"),
    "-I", CSRC,
]


def build(verbose: bool = False, extra_flags=(), out: str = LIB) -> str:
    srcs = [os.path.join(CSRC, s) for s in SOURCES]
    tmp = out + ".tmp"
    cmd = [HIPCC, *FLAGS, *extra_flags, *srcs, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        sys.stderr.write(r.stdout + r.stderr)
        raise RuntimeError("hipcc failed building libattn.so")
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    print(build(verbose=True))
