"""Build libripe.so (the C-ABI library) for gfx950 with hipcc, in-tree.

Usage: ``python self_speculative_verify_ripe_amd/build.py`` (or ``build()``); run it as a
script, since importing the package loads the library it is about to rebuild.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libripe.so")
# bench.py's read-floor context: its own library, never loaded by the binding
FLOOR_SRC = os.path.join(PKG, "measure", "read_floor.hip")
FLOOR_LIB = os.path.join(PKG, "measure", "libripe_readfloor.so")
SOURCES = ("api.hip", "verify.hip", "commit.hip", "accept.hip", "side_stats.hip")
ARCH = os.environ.get("RIPE_OFFLOAD_ARCH", "gfx950")


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found")


def _compile(sources, out: str, verbose: bool) -> str:
    tmp = out + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-shared",
           "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
           "-Wall", "-Wno-unused-result", "-I", INCLUDE, "-I", CSRC, "-o", tmp]
    cmd += list(sources)
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    noise = "is not a recognized feature for this target"
    msgs = [ln for ln in (res.stdout + res.stderr).splitlines() if noise not in ln]
    if res.returncode != 0:
        raise RuntimeError("hipcc failed:\n" + "\n".join(msgs))
    if verbose and msgs:
        print("\n".join(msgs), flush=True)
    os.replace(tmp, out)
    return out


def build(verbose: bool = False) -> str:
    """Compile every source into libripe.so, and the bench's read-floor
    library beside it (always recompiles)."""
    _compile([os.path.join(CSRC, s) for s in SOURCES], LIB, verbose)
    _compile([FLOOR_SRC], FLOOR_LIB, verbose)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
