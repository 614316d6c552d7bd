"""Build the gfx950 shared library ``libw4a16.so`` in-tree with hipcc.

Usage: ``python -m w4a16_gemm_amd.build`` (or ``__graft_entry__.build()``).
Every HIP translation unit is compiled for gfx950 only, with packed fp32 VALU ops
disabled (``-packed-fp32-ops``); objects go to ``w4a16_gemm_amd/_build/`` and the
library to ``w4a16_gemm_amd/libw4a16.so``.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libw4a16.so")
SOURCES = ["api.cpp", "pack.hip", "layout.hip", "ceilings.hip", "noalloc.hip", "skinny.hip", "gemm.hip", "w4a8.hip"]
# Per-file flags.  The skinny kernels keep their few MFMA accumulators in VGPRs (the
# per-group epilogue reads them with plain VALU operations instead of v_accvgpr_read).
EXTRA = {"skinny.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"]}

HIPCC = os.environ.get("HIPCC", shutil.which("hipcc") or "/opt/rocm/bin/hipcc")
COMMON = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-fhip-fp32-correctly-rounded-divide-sqrt",
    "-Wall", "-Wno-unused-function",
    "-I", os.path.join(ROOT, "include"),
]


def _run(cmd):
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    out = "\n".join(l for l in r.stdout.splitlines() if "packed-fp32-ops" not in l)
    return r.returncode, out


def build(verbose: bool = False, jobs: int = 8) -> str:
    os.makedirs(BUILD, exist_ok=True)
    objs, cmds = [], []
    for src in SOURCES:
        obj = os.path.join(BUILD, src + ".o")
        objs.append(obj)
        cmds.append([HIPCC, *COMMON, *EXTRA.get(src, []), "-c", os.path.join(CSRC, src), "-o", obj])
    with cf.ThreadPoolExecutor(max_workers=min(jobs, len(cmds))) as ex:
        results = list(ex.map(_run, cmds))
    for cmd, (rc, out) in zip(cmds, results):
        if verbose or rc != 0:
            if out.strip():
                print(out, file=sys.stderr)
        if rc != 0:
            raise RuntimeError(f"hipcc failed ({rc}): {' '.join(cmd)}")
    tmp = LIB + ".tmp"
    rc, out = _run([HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp, *objs])
    if rc != 0:
        print(out, file=sys.stderr)
        raise RuntimeError("hipcc link failed")
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
