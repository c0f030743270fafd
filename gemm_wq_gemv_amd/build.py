"""Build libwqmm.so in-tree with hipcc for gfx950.

Usage: ``python gemm_wq_gemv_amd/build.py`` (or ``__graft_entry__.build()``); not
``python -m``, which would first import the package and load the old library.
Always recompiles.  Objects go to ``gemm_wq_gemv_amd/_build/``; the shared
library to ``gemm_wq_gemv_amd/libwqmm.so``.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
BUILD = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "libwqmm.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

SOURCES = ["wqmm_api.hip", "gemv.hip", "gemm.hip", "skinny.hip", "pack.hip", "topk.hip", "attn.hip", "probe.hip", "smallm.hip", "wstream.hip", "hgemm.hip"]

# gfx950 only.  Packed-FP32 VALU ops are disabled for all device code; the
# host pass does not know that target feature and warns, which is harmless.
HIPFLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-Wall", "-Wno-unused-function",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", os.path.join(ROOT, "include"),
]


def _run(cmd):
    p = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    out = "\n".join(line for line in p.stdout.splitlines()
                    if "packed-fp32-ops" not in line and "target feature" not in line
                    and line.strip() != "1 warning generated.")
    if p.returncode != 0:
        raise RuntimeError(f"command failed ({p.returncode}): {' '.join(cmd)}\n{p.stdout}")
    return out


# Per-file flags.  hgemm.hip: matrix-core results in ordinary VGPRs (the lane
# scales and adds them; without this the compiler keeps them in AGPRs and
# copies them back and forth every step).
FILE_FLAGS = {"hgemm.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"]}


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    objs = [os.path.join(BUILD, os.path.splitext(s)[0] + ".o") for s in SOURCES]
    cmds = [[HIPCC, *HIPFLAGS, *FILE_FLAGS.get(s, []), "-c", os.path.join(CSRC, s), "-o", o]
            for s, o in zip(SOURCES, objs)]
    with cf.ThreadPoolExecutor(max_workers=min(len(cmds), 8)) as ex:
        for out in ex.map(_run, cmds):
            if verbose and out.strip():
                print(out)
    tmp = LIB + ".tmp"
    _run([HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp, *objs])
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
