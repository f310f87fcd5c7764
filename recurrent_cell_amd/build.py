"""Compile the HIP library libcfc.so for gfx950 (in-tree, next to this file).

hipcc builds the kernels and the C-ABI host layer in one shared object.  All
device code is built with packed-fp32 instructions disabled: the compiler
would otherwise emit v_pk_* fp32 forms by itself.
"""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
SOURCES = [os.path.join(HERE, "csrc", f) for f in ("cfc_kernels.hip", "cfc_api.hip", "gemm_kernels.hip",
                                                    "mlp_api.hip", "probe.hip")]
HEADERS = [os.path.join(HERE, "csrc", f) for f in ("cfc_kernels.h", "cfc_math.h", "api_common.h", "gemm_kernels.h")] + \
    [os.path.join(ROOT, "include", f) for f in ("cfc.h", "mlp.h", "probe.h")]
LIB = os.path.join(HERE, "libcfc.so")
ARCH = "gfx950"

HIPCC_FLAGS = [
    "-O3", "-std=c++17", "-fPIC", "-shared", "--offload-arch=" + ARCH,
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-command-line-argument",
    "-I", os.path.join(ROOT, "include"),
]


def hipcc() -> str:
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    path = os.path.join(rocm, "bin", "hipcc")
    return path if os.path.exists(path) else "hipcc"


def build(force: bool = True, verbose: bool = False) -> str:
    """Compile libcfc.so; with force=False, skip when it is newer than every source."""
    if not force and os.path.exists(LIB):
        newest = max(os.path.getmtime(p) for p in SOURCES + HEADERS)
        if os.path.getmtime(LIB) >= newest:
            return LIB
    tmp = LIB + ".tmp%d" % os.getpid()
    cmd = [hipcc()] + HIPCC_FLAGS + ["-o", tmp] + SOURCES
    if verbose:
        print(" ".join(cmd))
    subprocess.run(cmd, check=True, cwd=HERE)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
