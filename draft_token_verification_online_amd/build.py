"""Build libspec_verify.so for gfx950 with hipcc (in-tree, no JIT cache)."""
from __future__ import annotations

import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
LIB = os.path.join(PKG, "libspec_verify.so")
SOURCES = [os.path.join(CSRC, "spec_verify.hip")]
DEPS = SOURCES + [os.path.join(CSRC, f) for f in ("sv_device.hpp", "sv_rowstats.hpp",
                                                  "sv_walk.hpp", "sv_spectr.hpp",
                                                  "sv_draft.hpp", "sv_lmhead.hpp",
                                                  "sv_single.hpp", "sv_redo.hpp")] + \
    [os.path.join(ROOT, "include", "spec_verify.h")]

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
    # code object v5: loadable by the HIP runtime that PyTorch bundles
    "-mcode-object-version=5",
    # keep the compiler from forming packed fp32 ops (v_pk_*_f32)
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function",
]


def build(verbose: bool = False) -> str:
    tmp = LIB + ".tmp"
    cmd = [HIPCC, *FLAGS, "-o", tmp, *SOURCES]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.check_call(cmd)
    os.replace(tmp, LIB)
    return LIB


def stale() -> bool:
    if not os.path.exists(LIB):
        return True
    t = os.path.getmtime(LIB)
    return any(os.path.getmtime(p) > t for p in DEPS)


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
