"""Build the C-ABI shared library ``libgqa_attn.so`` for gfx950 with hipcc.

Usage: ``python -m attention_gqa_causal_amd.build [--debug]`` (or ``build()``
from Python).  The library is written next to this file so that it travels
with the source tree; objects go to ``_build/`` at the repository root.

``--debug`` (``build(debug=True)``) builds ``libgqa_attn_debug.so`` instead:
the same kernels compiled with GQA_DEBUG, which record every kind of device-side
metadata they had to clamp (read back with ``gqa_attn_debug_flags``).  Point
``GQA_ATTN_LIB`` at it to use it from the Python binding.
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
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libgqa_attn.so")
LIB_DEBUG = os.path.join(PKG, "libgqa_attn_debug.so")

SOURCES = ["api.cpp", "prefill_bf16.hip", "decode_bf16.hip", "generic_fp32.hip", "ring.hip", "rope.hip", "backward.hip",
           "decode_step.hip"]
ARCH = "gfx950"


def hipcc() -> str:
    return os.environ.get("HIPCC") or shutil.which("hipcc") or "/opt/rocm/bin/hipcc"


def common_flags():
    return [
        f"--offload-arch={ARCH}",
        "-O3",
        "-std=c++17",
        "-fPIC",
        "-ffp-contract=fast",
        # no packed-fp32 VALU instructions in device code
        "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
        "-I", INCLUDE,
        "-I", CSRC,
    ]


def _compile(src: str, debug: bool = False) -> str:
    obj = os.path.join(BUILD, "debug" if debug else "", os.path.splitext(src)[0] + ".o")
    cmd = [hipcc(), "-x", "hip", "-c", os.path.join(CSRC, src), "-o", obj] + common_flags()
    if debug:
        cmd.append("-DGQA_DEBUG")
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    return obj


def build(verbose: bool = False, debug: bool = False) -> str:
    os.makedirs(os.path.join(BUILD, "debug"), exist_ok=True)
    with cf.ThreadPoolExecutor(max_workers=min(4, len(SOURCES))) as ex:
        objs = list(ex.map(lambda src: _compile(src, debug), SOURCES))
    lib = LIB_DEBUG if debug else LIB
    tmp = lib + ".tmp"
    cmd = [hipcc(), "-shared", "-fPIC", f"--offload-arch={ARCH}", "-o", tmp] + objs
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, lib)
    if verbose:
        print(f"built {lib}")
    return lib


if __name__ == "__main__":
    build(verbose=True, debug="--debug" in sys.argv[1:])
    sys.exit(0)
