"""Build libgdn_cpr.so in-tree for gfx950 with hipcc.

    python -m bitwise_invariant_gated_amd.build

Flags that fix the numerics: -ffp-contract=off (every FMA in the library is
written explicitly), no fast-math, and packed-fp32 instructions disabled for
the device code.
"""

from __future__ import annotations

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
SRC = os.path.join(HERE, "csrc", "gdn_cpr.hip")
OUT = os.path.join(HERE, "libgdn_cpr.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

FLAGS = [
    "--offload-arch=gfx950",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-shared",
    "-ffp-contract=off",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", os.path.join(ROOT, "include"),
]


def build(verbose: bool = True) -> str:
    tmp = OUT + ".tmp"
    cmd = [HIPCC, *FLAGS, "-o", tmp, SRC]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    # the host pass does not know the packed-fp32 target feature; that warning is expected
    lines = [ln for ln in (res.stdout + res.stderr).splitlines() if "packed-fp32-ops" not in ln
             and ln.strip() and not ln.startswith("1 warning")]
    if res.returncode != 0:
        sys.stderr.write("\n".join(lines) + "\n")
        raise RuntimeError(f"hipcc failed with status {res.returncode}")
    if verbose and lines:
        print("\n".join(lines))
    os.replace(tmp, OUT)
    return OUT


if __name__ == "__main__":
    build()
