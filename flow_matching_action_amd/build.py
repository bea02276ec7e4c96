"""Build libpi_ae.so (gfx950) in-tree with hipcc.

Usage: python -m flow_matching_action_amd.build
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libpi_ae.so")
SOURCES = [os.path.join(CSRC, "pi_ae_kernels.hip"), os.path.join(CSRC, "pi_ae_diag.hip"),
           os.path.join(CSRC, "pi_ae_noalloc.hip"), os.path.join(CSRC, "pi_ae_runtime.cpp")]

# Packed-fp32 VALU forms are kept out of generated code on purpose.  MFMA
# results go to ordinary VGPRs: the attention kernels rescale their
# accumulators with VALU code, which on accumulation registers costs a copy of
# every accumulator out and back each step.
HIP_FLAGS = ["--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-fvisibility=hidden",
             "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
             "-mllvm", "-amdgpu-mfma-vgpr-form"]


def hipcc() -> str:
    for cand in (shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm toolchain required to build libpi_ae.so)")


# Host-side AddressSanitizer and UndefinedBehaviorSanitizer for the runtime's
# host code (argument checks, fp64 preparation, graph cache); each -fsanitize
# applies to the host compilation only (GPU code is built as usual).
SANITIZE_FLAGS = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
                  "-Xarch_host", "-fno-sanitize-recover=undefined", "-Xarch_host", "-fno-omit-frame-pointer",
                  "-shared-libsan", "-g"]


def sanitizer_runtime() -> str:
    """The shared ASan runtime a non-instrumented interpreter must preload to load a sanitized build."""
    res = subprocess.run([hipcc(), "--print-file-name=libclang_rt.asan-x86_64.so"], capture_output=True, text=True)
    path = res.stdout.strip()
    if not os.path.isabs(path) or not os.path.exists(path):
        raise RuntimeError("the clang ASan runtime (libclang_rt.asan-x86_64.so) was not found")
    return path


def build(verbose: bool = False, sanitize: bool = False, out: str | None = None) -> str:
    """Compile every source into flow_matching_action_amd/libpi_ae.so (or `out`);
    returns its path.  sanitize: host code built with ASan + UBSan."""
    lib = out or LIB
    tmp = lib + ".tmp"
    cmd = [hipcc(), *HIP_FLAGS, *(SANITIZE_FLAGS if sanitize else []), "-shared", "-I", os.path.join(ROOT, "include"),
           "-I", CSRC, "-o", tmp, *SOURCES]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        sys.stderr.write(res.stdout + res.stderr)
        raise RuntimeError(f"hipcc failed with exit code {res.returncode}")
    os.replace(tmp, lib)
    return lib


if __name__ == "__main__":
    print(build(verbose=True))
