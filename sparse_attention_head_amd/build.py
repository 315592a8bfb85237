"""Builds libdsa.so (HIP kernels + C ABI) for gfx950 in-tree with hipcc.

    python sparse_attention_head_amd/build.py [-v]

(run as a script: importing the package would load the library before it is rebuilt)

Every call recompiles all sources. Objects go to <repo>/_build/, the library to
sparse_attention_head_amd/libdsa.so.
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
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libdsa.so")

SOURCES = ["dsa_api.cpp", "indexer.hip", "topk.hip", "attn.hip"]
ARCH = os.environ.get("DSA_OFFLOAD_ARCH", "gfx950")

COMMON = ["-O3", "-std=c++17", "-fPIC", f"-I{INCLUDE}", f"-I{CSRC}", "-Wall", "-Wno-unused-function"]
# packed fp32 instructions are kept out of the device code
DEVICE = [f"--offload-arch={ARCH}", "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
          "-munsafe-fp-atomics"]


def hipcc():
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc"):
        if c and os.path.exists(c):
            return c
    return "hipcc"


# per-file code generation options: the indexer consumes every matrix-instruction result with
# vector instructions, so its MFMAs write the architectural registers directly
PER_FILE = {"indexer.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"]}


def _compile(src, verbose):
    obj = os.path.join(BUILD, src + ".o")
    cmd = [hipcc(), *COMMON, *DEVICE, *PER_FILE.get(src, []), "-x", "hip", "-c", os.path.join(CSRC, src),
           "-o", obj]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{r.stdout}\n{r.stderr}")
    if verbose and r.stderr.strip():
        print(r.stderr, file=sys.stderr)
    return obj


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    with ThreadPoolExecutor(len(SOURCES)) as ex:
        objs = list(ex.map(lambda s: _compile(s, verbose), SOURCES))
    tmp = LIB + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
