"""Build libhla_san.so: the library with AddressSanitizer and UndefinedBehaviorSanitizer
on its host code (argument validation, workspace sizing, the RoPE table helper, launch
set-up), for CPU-only checks of the C ABI. Device code is built as usual.

    python -m softmax_attention_relu_amd.build_sanitize

Load it with the shared sanitizer runtime preloaded, e.g.

    LD_PRELOAD=$(python -m softmax_attention_relu_amd.build_sanitize --runtime) \\
    ASAN_OPTIONS=detect_leaks=0 HLA_LIBRARY=softmax_attention_relu_amd/libhla_san.so \\
    python -m pytest tests/test_abi_host.py
"""
from __future__ import annotations

import glob
import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

from .build import ARCH, CSRC, DEVICE_FLAGS, FLAGS, HIPCC, PKG, ROOT, SOURCES

SAN_BUILD = os.path.join(ROOT, "_build", "san")
SAN_LIB = os.path.join(PKG, "libhla_san.so")
# each sanitizer flag right after -Xarch_host: host code only
HOST_SAN = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
            "-Xarch_host", "-fno-sanitize-recover=undefined", "-Xarch_host", "-fno-omit-frame-pointer"]


def runtime() -> str:
    """Path of the shared AddressSanitizer runtime of the ROCm compiler."""
    hits = sorted(glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
    if not hits:
        raise FileNotFoundError("libclang_rt.asan-x86_64.so not found under /opt/rocm/llvm")
    return hits[-1]


def _compile(src: str) -> str:
    obj = os.path.join(SAN_BUILD, os.path.splitext(src)[0] + ".o")
    cmd = [HIPCC, *FLAGS, *DEVICE_FLAGS.get(src, []), *HOST_SAN, "-c", os.path.join(CSRC, src), "-o", obj]
    if src.endswith(".cpp"):
        cmd[1:1] = ["-x", "hip"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stderr}")
    return obj


def build() -> str:
    os.makedirs(SAN_BUILD, exist_ok=True)
    with ThreadPoolExecutor(len(SOURCES)) as ex:
        objs = list(ex.map(_compile, SOURCES))
    tmp = SAN_LIB + ".tmp"
    r = subprocess.run([HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-Xarch_host", "-fsanitize=address",
                        "-Xarch_host", "-fsanitize=undefined", "-shared-libsan", *objs, "-o", tmp],
                       capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr}")
    os.replace(tmp, SAN_LIB)
    return SAN_LIB


if __name__ == "__main__":
    if "--runtime" in sys.argv[1:]:
        print(runtime())
    else:
        print(f"built {build()}")
