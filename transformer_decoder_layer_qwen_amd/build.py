"""Build the layer library ``libqlayer.so`` in-tree for gfx950.

Every ``csrc/*.hip`` file is compiled with hipcc for ``--offload-arch=gfx950``
(packed-fp32 instructions disabled), ``csrc/qlayer.cpp`` as host C++, and the
objects are linked into ``libqlayer.so`` next to this file. Run
``python -m transformer_decoder_layer_qwen_amd.build`` or call ``build()``.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(os.path.dirname(PKG), "include")
BUILD = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libqlayer.so")

ARCH = "gfx950"
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
DEVICE_FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-unused-result",
]
HOST_FLAGS = [f"--offload-arch={ARCH}", "-O2", "-std=c++17", "-fPIC"]
# Per-file device flags. gemm2.hip: MFMA results in the ordinary vector
# registers, so the decode tiles' accumulators, which also feed stores and
# selects, are not copied between register files at every k step.
FILE_FLAGS = {"gemm2.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"]}


def _run(cmd):
    p = subprocess.run(cmd, capture_output=True, text=True)
    if p.returncode != 0:
        raise RuntimeError(f"command failed ({p.returncode}): {' '.join(cmd)}\n{p.stdout}\n{p.stderr}")
    return p


def build(verbose: bool = False, jobs: int = 8) -> str:
    """Compile every source and link the shared library; returns its path."""
    if not os.path.exists(HIPCC):
        raise RuntimeError(f"hipcc not found at {HIPCC}")
    os.makedirs(BUILD, exist_ok=True)
    srcs = sorted(f for f in os.listdir(CSRC) if f.endswith((".hip", ".cpp")))
    cmds = []
    objs = []
    for f in srcs:
        src = os.path.join(CSRC, f)
        obj = os.path.join(BUILD, f + ".o")
        objs.append(obj)
        if f.endswith(".hip"):
            cmds.append([HIPCC, *DEVICE_FLAGS, *FILE_FLAGS.get(f, []), f"-I{INCLUDE}", "-c", src,
                         "-o", obj])
        else:
            cmds.append([HIPCC, *HOST_FLAGS, f"-I{INCLUDE}", "-c", src, "-o", obj])
    with cf.ThreadPoolExecutor(max_workers=max(1, jobs)) as ex:
        futs = {ex.submit(_run, c): c for c in cmds}
        for fu in cf.as_completed(futs):
            fu.result()
            if verbose:
                print("compiled", futs[fu][-3])
    tmp = LIB + ".tmp"
    _run([HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs])
    os.replace(tmp, LIB)
    if verbose:
        print("linked", LIB)
    return LIB


def clean() -> None:
    shutil.rmtree(BUILD, ignore_errors=True)
    if os.path.exists(LIB):
        os.remove(LIB)


if __name__ == "__main__":
    build(verbose=True, jobs=int(os.environ.get("MAX_JOBS", "8")))
    sys.exit(0)
