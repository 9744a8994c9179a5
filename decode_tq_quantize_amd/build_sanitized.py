"""Host-sanitized build of libtq for the CPU checks of the C ABI layer.

    python -m decode_tq_quantize_amd.build_sanitized

The host-only sources (argument validation, workspace sizing, the fp64
Lloyd-Max builder) are compiled by g++ with AddressSanitizer and
UndefinedBehaviorSanitizer and linked with the regular objects of the kernel
sources into _build/san/libtq_san.so. The tests load it through the
TQ_LIBRARY variable with the sanitizer runtimes preloaded (an uninstrumented
python cannot load them later). Device code is not instrumented.
"""
from __future__ import annotations

import os
import subprocess

from . import build as _b

SAN_DIR = os.path.join(_b.OBJDIR, "san")
OUT = os.path.join(SAN_DIR, "libtq_san.so")
HOST_SOURCES = ["codebook.cpp", "tq_api.cpp"]
SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=undefined", "-fno-omit-frame-pointer"]


def runtime_preload() -> str:
    """LD_PRELOAD value naming gcc's ASan and UBSan runtimes."""
    libs = []
    for name in ("libasan.so", "libubsan.so"):
        libs.append(subprocess.run(["gcc", f"-print-file-name={name}"], capture_output=True, text=True,
                                   check=True).stdout.strip())
    return ":".join(libs)


def build_sanitized() -> str:
    kernel_objs = [os.path.join(_b.OBJDIR, os.path.splitext(s)[0] + ".o") for s in _b.SOURCES
                   if s not in HOST_SOURCES]
    if not all(os.path.exists(o) for o in kernel_objs):
        _b.build(verbose=False)
    os.makedirs(SAN_DIR, exist_ok=True)
    objs = []
    for src in HOST_SOURCES:
        obj = os.path.join(SAN_DIR, os.path.splitext(src)[0] + ".o")
        cmd = ["g++", "-O1", "-g", "-std=c++17", "-fPIC", *SAN, "-D__HIP_PLATFORM_AMD__", "-I/opt/rocm/include",
               "-I" + _b.INCLUDE, "-I" + _b.CSRC, "-c", os.path.join(_b.CSRC, src), "-o", obj]
        subprocess.run(cmd, check=True, capture_output=True, text=True)
        objs.append(obj)
    cmd = ["g++", "-shared", *SAN[:1], *objs, *kernel_objs, "-L/opt/rocm/lib", "-lamdhip64",
           "-Wl,-rpath,/opt/rocm/lib", "-o", OUT]
    subprocess.run(cmd, check=True, capture_output=True, text=True)
    return OUT


if __name__ == "__main__":
    print(build_sanitized())
