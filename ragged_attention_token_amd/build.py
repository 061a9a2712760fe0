"""Build librag.so (HIP, gfx950) in-tree with hipcc.

    python -m ragged_attention_token_amd.build

Every HIP source is compiled for gfx950 only, with packed-fp32 instruction
selection switched off (-Xclang -target-feature -Xclang -packed-fp32-ops) and
MFMA operands kept in VGPRs (-mllvm -amdgpu-mfma-vgpr-form); the
HIP-free validation unit is compiled as plain C++17.  The result lands next to
this file, where the binding loads it.
"""
from __future__ import annotations

import glob
import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(HERE, "librag.so")
ARCH = "gfx950"

HIP_FLAGS = [
    "-O3", "-std=c++17", "-fPIC", "--offload-arch=" + ARCH,
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # keep MFMA accumulators in ordinary VGPRs (no AGPR <-> VGPR copies around
    # the fp32 softmax updates of the accumulator)
    "-mllvm", "-amdgpu-mfma-vgpr-form",
    # no kernel relies on NaN semantics; this lets fmaxf map to a bare v_max
    # (no quieting of its inputs) in the softmax's row maxima
    "-fno-honor-nans",
    "-fvisibility=hidden", "-DRAG_BUILDING_LIBRARY", "-I" + INCLUDE, "-I" + CSRC,
    "-Wall", "-Werror", "-Wno-unused-command-line-argument",
]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found: the HIP library cannot be built")


def sources():
    return sorted(glob.glob(os.path.join(CSRC, "*.hip"))) + sorted(glob.glob(os.path.join(CSRC, "*.cpp")))


def build(verbose: bool = False) -> str:
    """Compile every source in csrc/ into librag.so (always recompiles)."""
    objdir = os.path.join(ROOT, "_build", "obj")
    os.makedirs(objdir, exist_ok=True)
    cc = hipcc()
    objs = []
    for src in sources():
        obj = os.path.join(objdir, os.path.basename(src) + ".o")
        if src.endswith(".hip"):
            cmd = [cc] + HIP_FLAGS + ["-x", "hip", "-c", src, "-o", obj]
        else:
            cmd = ["g++", "-O2", "-std=c++17", "-fPIC", "-fvisibility=hidden",
                   "-DRAG_BUILDING_LIBRARY", "-I" + INCLUDE, "-I" + CSRC, "-Wall", "-Wextra",
                   "-Werror", "-c", src, "-o", obj]
        if verbose:
            print(" ".join(cmd), flush=True)
        res = subprocess.run(cmd, capture_output=True, text=True)
        noise = "is not a recognized feature for this target"
        err = "\n".join(l for l in res.stderr.splitlines() if noise not in l)
        if res.returncode != 0:
            raise RuntimeError("compile failed: %s\n%s" % (" ".join(cmd), err))
        if err.strip() and verbose:
            print(err)
        objs.append(obj)
    tmp = LIB + ".tmp%d" % os.getpid()
    # --no-undefined: a kernel whose host stub clang failed to emit would
    # otherwise only surface when the library is loaded
    cmd = [cc, "-shared", "-fPIC", "--offload-arch=" + ARCH, "-Wl,--no-undefined", "-o", tmp] + objs
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError("link failed: %s\n%s" % (" ".join(cmd), res.stderr))
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
