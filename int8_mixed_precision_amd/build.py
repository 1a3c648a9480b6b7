"""Build the HIP library (libkv4.so) for gfx950 with hipcc.

Run ``python -m int8_mixed_precision_amd.build``; ``__graft_entry__.build()``
calls :func:`build`.  The library is built in-tree next to this file.
"""
from __future__ import annotations

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
SRC = os.path.join(HERE, "csrc", "kv4.hip")
LIB = os.path.join(HERE, "libkv4.so")
# read-bandwidth ceilings (measurement aid, include/kv4_roof.h)
ROOF_SRC = os.path.join(HERE, "csrc", "kv4_roof.hip")
ROOF_LIB = os.path.join(HERE, "libkv4_roof.so")
# the same library with the device-side checks of KV4_VALIDATE (include/kv4.h)
VALIDATE_LIB = os.path.join(HERE, "libkv4_validate.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

HIPFLAGS = [
    "--offload-arch=gfx950",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-shared",
    # packed fp32 instructions are kept out of the generated code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # MFMA accumulators in ordinary VGPRs: the decode loops then need no
    # accumulator-register copies
    "-mllvm", "-amdgpu-mfma-vgpr-form",
    "-Wall",
    "-Wno-unused-function",
    "-I", os.path.join(ROOT, "include"),
]


def sources():
    """Sources of the decode library (libkv4.so)."""
    csrc = os.path.join(HERE, "csrc")
    return [os.path.join(csrc, f) for f in sorted(os.listdir(csrc))
            if f.endswith((".hip", ".hpp", ".h")) and f != "kv4_roof.hip"] + \
        [os.path.join(ROOT, "include", "kv4.h")]


def _compile(src, lib, verbose, extra=()):
    tmp = lib + ".tmp"
    cmd = [HIPCC, *HIPFLAGS, *extra, src, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.check_call(cmd)
    os.replace(tmp, lib)


def build(verbose: bool = False) -> str:
    """Compiles the library, its validating build and the read-ceiling
    kernels (three independent hipcc runs, in parallel)."""
    from concurrent.futures import ThreadPoolExecutor
    jobs = [(SRC, LIB, ()), (SRC, VALIDATE_LIB, ("-DKV4_VALIDATE",)), (ROOF_SRC, ROOF_LIB, ())]
    with ThreadPoolExecutor(len(jobs)) as ex:
        for f in [ex.submit(_compile, src, lib, verbose, extra) for src, lib, extra in jobs]:
            f.result()
    return LIB


if __name__ == "__main__":
    build(verbose="-v" in sys.argv)
    print(LIB)
