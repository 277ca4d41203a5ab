"""Host-side sanitizer build of libhstu, for CPU tests only.

    python -m hstu_jagged_pointwise_amd.asan_build

The host code of api.cpp (argument validation, workspace carving, launch order) is
compiled with AddressSanitizer and UndefinedBehaviorSanitizer, on the host compilation
only (each flag behind -Xarch_host); device code is built as usual. The other objects
come from the regular build. The shared library lands at _build/asan/libhstu_asan.so and
needs the shared ASan runtime (asan_runtime()) preloaded into the process that loads it.
No GPU run uses this build.
"""
from __future__ import annotations

import os
import subprocess
import sys

from hstu_jagged_pointwise_amd import build as B

ASAN_DIR = os.path.join(B.BUILD, "asan")
ASAN_LIB = os.path.join(ASAN_DIR, "libhstu_asan.so")
LLVM_BIN = os.path.join(os.path.dirname(os.path.realpath(B.HIPCC)), "..", "llvm", "bin")


def asan_runtime() -> str:
    clang = os.path.join(LLVM_BIN, "..", "lib", "clang")
    for ver in sorted(os.listdir(clang)) if os.path.isdir(clang) else []:
        rt = os.path.join(clang, ver, "lib", "linux", "libclang_rt.asan-x86_64.so")
        if os.path.exists(rt):
            return os.path.realpath(rt)
    raise RuntimeError("no shared ASan runtime under the ROCm LLVM")


def build_asan(verbose: bool = True) -> str:
    B.build(verbose=False)
    os.makedirs(ASAN_DIR, exist_ok=True)
    obj = os.path.join(ASAN_DIR, "api.o")
    host_san = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
                "-Xarch_host", "-fno-sanitize-recover=all", "-Xarch_host", "-fno-omit-frame-pointer"]
    cmd = [B.HIPCC, *B.COMMON, "-g", *host_san, "-x", "hip", "-c",
           os.path.join(B.CSRC, "api.cpp"), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc (sanitized host code) failed on api.cpp:\n{r.stderr}")
    objs = [obj] + [os.path.join(B.BUILD, os.path.splitext(f)[0] + ".o") for f in B.SOURCES
                    if f != "api.cpp"]
    # host link (each object already embeds its device code) with the shared ASan runtime
    rocm_lib = os.path.realpath(os.path.join(os.path.dirname(os.path.realpath(B.HIPCC)), "..", "lib"))
    tmp = ASAN_LIB + ".tmp"
    link = [os.path.join(LLVM_BIN, "clang++"), "-shared", "-fPIC", "-shared-libasan",
            "-fsanitize=address,undefined", "-o", tmp, *objs, f"-L{rocm_lib}",
            f"-Wl,-rpath,{rocm_lib}", "-lamdhip64"]
    r = subprocess.run(link, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link (sanitized host code) failed:\n{r.stderr}")
    os.replace(tmp, ASAN_LIB)
    if verbose:
        print(f"built {ASAN_LIB}")
    return ASAN_LIB


if __name__ == "__main__":
    try:
        build_asan()
    except RuntimeError as e:
        print(e, file=sys.stderr)
        sys.exit(1)
