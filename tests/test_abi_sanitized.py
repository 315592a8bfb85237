"""The host side of the C ABI under AddressSanitizer and UndefinedBehaviorSanitizer (no GPU).

Builds the library with the sanitizers on its host code only (the kernels are compiled as
usual), links the C driver tests/sanitize/abi_driver.c against it with the same sanitizers, and
runs it: the driver walks every entry point's validation and size queries; any wrong status or
sanitizer report fails the test."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "sparse_attention_head_amd", "csrc")
INCLUDE = os.path.join(ROOT, "include")
OUT = os.path.join(ROOT, "_build", "sanitize")
ROCM = "/opt/rocm"
HIPCC = os.path.join(ROCM, "bin", "hipcc")
CLANG = os.path.join(ROCM, "llvm", "bin", "clang")

pytestmark = pytest.mark.skipif(not (os.path.exists(HIPCC) and os.path.exists(CLANG)),
                                reason="ROCm compilers not found")

# host-code sanitizers only: each -fsanitize goes after -Xarch_host on the hipcc lines
SAN_HOST = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
            "-Xarch_host", "-fno-sanitize-recover=undefined"]
SAN = ["-fsanitize=address", "-fsanitize=undefined", "-fno-sanitize-recover=undefined"]


def _run(cmd, **kw):
    r = subprocess.run(cmd, capture_output=True, text=True, **kw)
    assert r.returncode == 0, f"{' '.join(cmd)}\n{r.stdout}\n{r.stderr}"
    return r


def test_abi_host_code_under_sanitizers():
    os.makedirs(OUT, exist_ok=True)
    common = ["-O1", "-g", "-std=c++17", "-fPIC", f"-I{INCLUDE}", f"-I{CSRC}", "--offload-arch=gfx950",
              "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]
    objs = []
    for src in ("dsa_api.cpp", "indexer.hip", "topk.hip", "attn.hip"):
        obj = os.path.join(OUT, src + ".o")
        extra = ["-mllvm", "-amdgpu-mfma-vgpr-form"] if src == "indexer.hip" else []
        _run([HIPCC, *common, *SAN_HOST, *extra, "-x", "hip", "-c", os.path.join(CSRC, src), "-o", obj])
        objs.append(obj)
    lib = os.path.join(OUT, "libdsa_san.so")
    _run([HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", *SAN_HOST, *objs, "-o", lib])
    exe = os.path.join(OUT, "abi_driver")
    _run([CLANG, "-O1", "-g", *SAN, f"-I{INCLUDE}", os.path.join(ROOT, "tests", "sanitize", "abi_driver.c"),
          lib, f"-Wl,-rpath,{OUT}", f"-Wl,-rpath,{ROCM}/lib", "-o", exe])
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=0",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    r = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=300)
    assert r.returncode == 0, f"driver failed ({r.returncode}):\n{r.stdout}\n{r.stderr}"
    assert "ERROR: AddressSanitizer" not in r.stderr and "runtime error" not in r.stderr, r.stderr
    assert "all checks passed" in r.stdout
