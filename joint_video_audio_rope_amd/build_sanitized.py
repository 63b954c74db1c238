"""A host-sanitized build of libmmdit.so, for CPU tests of the C ABI.

abi.hip (argument checks, workspace plans, the RoPE table, dispatch) has its
host code built with AddressSanitizer and UndefinedBehaviorSanitizer (the
device code is untouched: the sanitizer flags are host-only); the kernels'
translation units are built as usual.  The result never runs on a GPU: the
tests load it into a CPU-only process with the ASan runtime preloaded and run
the ABI's host-side tests against it.

Usage: python -m joint_video_audio_rope_amd.build_sanitized
"""
import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

from . import build as B

OUT = os.path.join(B.BUILD, "sanitized")
LIB = os.path.join(OUT, "libmmdit_sanitized.so")
HOST_SANITIZE = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
                 "-Xarch_host", "-fno-sanitize-recover=undefined", "-Xarch_host", "-fno-omit-frame-pointer"]


def asan_runtime():
    """Path of the clang ASan runtime that matches hipcc."""
    p = subprocess.run([B.hipcc(), "-print-file-name=libclang_rt.asan-x86_64.so"], stdout=subprocess.PIPE,
                       text=True, check=True).stdout.strip()
    if not os.path.exists(p):
        raise RuntimeError("ASan runtime not found (%s)" % p)
    return p


def build(jobs=4):
    cc = B.hipcc()
    os.makedirs(OUT, exist_ok=True)

    def one(src):
        obj = os.path.join(OUT, src.replace(".hip", ".o"))
        flags = B.HIPFLAGS + (HOST_SANITIZE + ["-g"] if src == "abi.hip" else [])
        B._run([cc] + flags + ["-c", os.path.join(B.CSRC, src), "-o", obj])
        return obj

    with ThreadPoolExecutor(max_workers=max(1, jobs)) as ex:
        objs = list(ex.map(one, B.SOURCES))
    B._run([cc, "--offload-arch=gfx950", "-shared", "-fPIC", "-shared-libasan", "-o", LIB] + objs + HOST_SANITIZE)
    return LIB


if __name__ == "__main__":
    print(build())
    sys.exit(0)
