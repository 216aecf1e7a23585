"""Builds libmsign.so in-tree with hipcc for gfx950.

The library is one translation unit (csrc/msign_api.hip includes the kernel
headers).  The output goes to a temporary file that is renamed into place, so
a failed build never leaves a half-written library behind.
"""

from __future__ import annotations

import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
SRC = os.path.join(HERE, "csrc", "msign_api.hip")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(HERE, "libmsign.so")
ARCH = "gfx950"

# Packed-fp32 instructions are kept out of the generated code on purpose.
FLAGS = ["-O3", "-std=c++17", "-fPIC", "-shared", f"--offload-arch={ARCH}",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-Wall", "-Wno-unused-function"]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (set HIPCC or install ROCm)")


def sources():
    csrc = os.path.join(HERE, "csrc")
    return [os.path.join(csrc, f) for f in sorted(os.listdir(csrc))
            if f.endswith((".hip", ".hpp", ".h"))] + [os.path.join(INCLUDE, "msign.h")]


def build(verbose: bool = False, extra_flags=None) -> str:
    tmp = LIB + ".tmp"
    cmd = [hipcc()] + FLAGS + list(extra_flags or []) + ["-I", INCLUDE, SRC, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        sys.stderr.write(res.stdout + res.stderr)
        if os.path.exists(tmp):
            os.remove(tmp)
        raise RuntimeError(f"hipcc failed with exit code {res.returncode}")
    noise = [ln for ln in (res.stdout + res.stderr).splitlines()
             if ln.strip() and "packed-fp32-ops" not in ln]
    if verbose and noise:
        sys.stderr.write("\n".join(noise) + "\n")
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
