"""Builds libmsign.so in-tree with hipcc for gfx950.

Each csrc/*.hip file is one translation unit (the host API, and the product
kernels for single and for grouped launches), compiled in parallel to
objects in a temporary folder and linked into one shared library.  The output
goes to a temporary file that is renamed into place, so a failed build never
leaves a half-written library behind.
"""

from __future__ import annotations

import os
import shutil
import subprocess
import sys
import tempfile

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(HERE, "libmsign.so")
ARCH = "gfx950"

# Packed-fp32 instructions are kept out of the generated code on purpose.
FLAGS = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
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


def translation_units():
    return [os.path.join(CSRC, f) for f in sorted(os.listdir(CSRC)) if f.endswith(".hip")]


def _run(cmds, verbose):
    """Run the commands in parallel; raise with the first failure's output."""
    procs = []
    for cmd in cmds:
        if verbose:
            print(" ".join(cmd), flush=True)
        procs.append(subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True))
    failed = None
    for cmd, p in zip(cmds, procs):
        out, _ = p.communicate()
        noise = [ln for ln in out.splitlines() if ln.strip() and "packed-fp32-ops" not in ln]
        if p.returncode != 0 and failed is None:
            failed = (p.returncode, out)
        elif verbose and noise:
            sys.stderr.write("\n".join(noise) + "\n")
    if failed:
        sys.stderr.write(failed[1])
        raise RuntimeError(f"hipcc failed with exit code {failed[0]}")


def build(verbose: bool = False, extra_flags=None) -> str:
    tmp = LIB + ".tmp"
    cc = hipcc()
    flags = FLAGS + list(extra_flags or []) + ["-I", INCLUDE]
    with tempfile.TemporaryDirectory(prefix="msign_build_") as objdir:
        objs, cmds = [], []
        for src in translation_units():
            obj = os.path.join(objdir, os.path.basename(src) + ".o")
            objs.append(obj)
            cmds.append([cc] + flags + ["-c", src, "-o", obj])
        try:
            _run(cmds, verbose)
            _run([[cc, "-shared", "-fPIC", f"--offload-arch={ARCH}"] + objs + ["-o", tmp]], verbose)
        except Exception:
            if os.path.exists(tmp):
                os.remove(tmp)
            raise
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
