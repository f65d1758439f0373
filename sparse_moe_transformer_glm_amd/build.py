"""Build ``libglm_moe.so`` (the layer, HIP, gfx950 only) and ``libglm_peaks.so``
(the hardware-ceiling microbenchmarks that ``bench.py`` runs) in-tree with hipcc.

Usage: ``python -m sparse_moe_transformer_glm_amd.build``.  Every call
recompiles; objects go to ``_build/`` at the repository root.
"""
from __future__ import annotations

import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libglm_moe.so")
SOURCES = ["router.hip", "permute.hip", "gemm_bf16.hip", "gemm_mx.hip", "gemm_f32.hip",
           "block.hip", "glm_moe.hip"]
PEAKS_LIB = os.path.join(PKG, "libglm_peaks.so")
PEAKS_SOURCES = ["peaks.hip"]
ARCH = "gfx950"


def hipcc() -> str:
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    return os.path.join(rocm, "bin", "hipcc")


def compile_flags():
    return [
        f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
        "-I", INCLUDE, "-I", CSRC,
        # keep the compiler from forming packed fp32 VALU ops
        "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
        "-fvisibility=hidden", "-Wno-unused-result",
    ]


def _run(cmd):
    r = subprocess.run(cmd, capture_output=True, text=True)
    noise = "is not a recognized feature for this target"
    err = "\n".join(l for l in r.stderr.splitlines() if noise not in l)
    if r.returncode != 0:
        raise RuntimeError(f"command failed ({r.returncode}): {' '.join(cmd)}\n{err}")
    return err


def build(verbose: bool = False) -> str:
    build_dir = os.path.join(ROOT, "_build")
    os.makedirs(build_dir, exist_ok=True)
    libs = ((LIB, SOURCES), (PEAKS_LIB, PEAKS_SOURCES))
    cmds, objs = [], {}
    for lib, sources in libs:
        for src in sources:
            obj = os.path.join(build_dir, src.replace(".hip", ".o"))
            objs.setdefault(lib, []).append(obj)
            cmds.append([hipcc(), *compile_flags(), "-c", os.path.join(CSRC, src), "-o", obj])
    with ThreadPoolExecutor(min(len(cmds), os.cpu_count() or 1)) as ex:
        for out in ex.map(_run, cmds):
            if verbose and out.strip():
                print(out, file=sys.stderr)
    for lib, _ in libs:
        tmp = lib + ".tmp"
        _run([hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs[lib], "-o", tmp])
        os.replace(tmp, lib)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
