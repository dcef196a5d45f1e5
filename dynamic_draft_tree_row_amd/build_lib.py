"""Compile the HIP sources into the in-tree shared library libddt.so (gfx950)."""
from __future__ import annotations

import os
import shutil
import subprocess
import tempfile

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libddt.so")
# (source, extra flags): the attention kernel assumes no NaNs and runs with
# the IEEE mode off, so that its float maxima need no operand canonicalisation
SOURCES = [
    ("ddt_api.hip", []),
    ("ddt_attention.hip", ["-fno-honor-nans", "-mno-amdgpu-ieee"]),
]
DEPS = ["ddt_api.hip", "ddt_attention.hip", "ddt_device.hpp", "ddt_rowreduce.hpp",
        "ddt_tree_kernels.hpp", "ddt_layer.hpp", "ddt_kvcache.hpp", "ddt_attention.hpp"]

HIPCC_FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
    # no packed fp32 instructions anywhere in the device code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
]


def hipcc() -> str:
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if c and os.path.exists(c):
            return c
    raise RuntimeError("hipcc not found; the draft-tree library needs ROCm's hipcc to build")


def _run(cmd, verbose):
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("hipcc failed:\n" + " ".join(cmd) + "\n" + r.stdout + r.stderr)
    if verbose and r.stderr.strip():
        print(r.stderr)


def build(verbose: bool = False) -> str:
    """Always recompiles; writes libddt.so next to this file and returns its path."""
    tmp = LIB + ".tmp"
    with tempfile.TemporaryDirectory() as d:
        objs = []
        for src, extra in SOURCES:
            obj = os.path.join(d, src + ".o")
            _run([hipcc(), *HIPCC_FLAGS, *extra, "-c", "-o", obj, os.path.join(CSRC, src)], verbose)
            objs.append(obj)
        _run([hipcc(), "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp, *objs], verbose)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
