"""Build the gfx950 shared library ``libadamw_amd.so`` in-tree with hipcc.

Usage: ``python adamw_optimizer_step_apply_amd/build.py`` (also run by
``__graft_entry__.build()``).  Run it as a script, not with ``-m``: importing
it as a submodule would first run the package's ``__init__``, which loads the
library this builds.  The library is written next to this file so that it
travels with the source tree.
"""
from __future__ import annotations

import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB_NAME = "libadamw_amd.so"
LIB_PATH = os.path.join(PKG, LIB_NAME)
SOURCES = ["kernels.hip", "plan.cpp", "validate.cpp", "api.cpp", "noalloc.hip"]
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

FLAGS = [
    "--offload-arch=gfx950",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-shared",
    # one binary32 operation per source operation: no fused multiply-add
    "-ffp-contract=off",
    # keep packed fp32 VALU instructions out of the generated code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall",
    "-Wno-unused-command-line-argument",
]


def build(verbose: bool = False) -> str:
    hipcc([os.path.join(CSRC, s) for s in SOURCES], LIB_PATH, verbose, include=[INCLUDE, CSRC])
    return LIB_PATH


def hipcc(srcs, out, verbose=False, include=()):
    """Compiles `srcs` into the shared library `out` for gfx950 with FLAGS."""
    tmp = out + ".tmp"
    inc = [a for d in include for a in ("-I", d)]
    cmd = [HIPCC, *FLAGS, *inc, "-o", tmp, *srcs]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        sys.stderr.write(r.stdout + r.stderr)
        raise RuntimeError(f"hipcc failed ({r.returncode}) building {os.path.basename(out)}")
    # the host pass does not know the gfx feature name; anything else is worth seeing
    noise = "'-packed-fp32-ops' is not a recognized feature for this target"
    rest = [ln for ln in (r.stdout + r.stderr).splitlines() if ln.strip() and noise not in ln]
    if rest:
        sys.stderr.write("\n".join(rest) + "\n")
    os.replace(tmp, out)


if __name__ == "__main__":
    print(build(verbose=True))
