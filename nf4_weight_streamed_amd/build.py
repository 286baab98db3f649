"""Build libnf4lora.so (the HIP library behind include/nf4lora.h) for gfx950.

Every source is compiled by hipcc into an object under _build/, then linked in
place as nf4_weight_streamed_amd/libnf4lora.so. Usage: python -m
nf4_weight_streamed_amd.build [-v]
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
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libnf4lora.so")

SOURCES = ["abi.cpp", "stream_pool.cpp", "nf4_codec.hip", "nf4_gemm_fwd.hip", "nf4_gemm_bwd.hip",
           "lora_skinny.hip", "nf4_skinny.hip", "stack_glue.hip",
           "probe.hip", "nf4_merge.hip", "noalloc.hip"]

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"
FLAGS = [
    "-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
    # packed fp32 instructions stay off in every kernel
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # float32 division in the quantiser must be correctly rounded
    "-fhip-fp32-correctly-rounded-divide-sqrt",
    "-Wall", "-Wno-unused-function",
]


def _compile(src: str, verbose: bool) -> str:
    obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
    lang = ["-x", "hip"] if src.endswith(".hip") else []
    cmd = [HIPCC, *FLAGS, *lang, "-c", os.path.join(CSRC, src), "-o", obj]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    errs = "\n".join(l for l in res.stderr.splitlines() if "packed-fp32-ops" not in l)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{errs}")
    if verbose and errs.strip():
        print(errs, flush=True)
    return obj


def build(verbose: bool = False) -> str:
    """Compile every source and link libnf4lora.so; returns its path. Always rebuilds."""
    if not os.path.exists(HIPCC):
        raise RuntimeError(f"hipcc not found at {HIPCC}")
    os.makedirs(BUILD, exist_ok=True)
    with cf.ThreadPoolExecutor(max_workers=min(8, len(SOURCES))) as ex:
        objs = list(ex.map(lambda s: _compile(s, verbose), SOURCES))
    tmp = LIB + ".tmp"
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"link failed:\n{res.stderr}")
    shutil.move(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
