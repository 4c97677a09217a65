"""Host-sanitizer build of libloglin.so for the CPU tests (not the product).

    python -m log_linear_token_amd.build_sanitized

Compiles every source as build.py does, with AddressSanitizer and
UndefinedBehaviorSanitizer on the host side of each translation unit only
(the gfx950 device code is built as usual), into _build/san/libloglin_san.so.
The library takes the sanitizer runtime from the process (LD_PRELOAD of
clang's libclang_rt.asan, which also carries the UBSan handlers); see
tests/test_host_sanitizers.py.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import subprocess
import sys

from log_linear_token_amd import build as B

OUT_DIR = os.path.join(B.BUILD, "san")
LIB = os.path.join(OUT_DIR, "libloglin_san.so")
HOST_SAN = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
            "-Xarch_host", "-fno-omit-frame-pointer", "-Xarch_host", "-fno-sanitize-recover=all",
            "-g1"]


def runtime() -> str:
    """clang's shared ASan runtime (with the UBSan handlers) matching hipcc."""
    clang = os.path.join(os.path.dirname(os.path.realpath(B.HIPCC)), "..", "lib", "llvm", "bin", "clang")
    if not os.path.exists(clang):
        clang = "/opt/rocm/llvm/bin/clang"
    return subprocess.check_output([clang, "-print-file-name=libclang_rt.asan-x86_64.so"], text=True).strip()


def _compile(src: str) -> str:
    obj = os.path.join(OUT_DIR, os.path.basename(src) + ".o")
    cmd = [B.HIPCC, *B.COMMON, *HOST_SAN, "-x", "hip", "-c", src, "-o", obj]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"compile failed: {' '.join(cmd)}\n{res.stdout}{res.stderr}")
    return obj


def build() -> str:
    os.makedirs(OUT_DIR, exist_ok=True)
    srcs = B.sources()
    with cf.ThreadPoolExecutor(min(len(srcs), 8)) as ex:
        objs = list(ex.map(_compile, srcs))
    tmp = LIB + ".tmp"
    cmd = [B.HIPCC, f"--offload-arch={B.ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"link failed: {' '.join(cmd)}\n{res.stdout}{res.stderr}")
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build())
    sys.exit(0)
