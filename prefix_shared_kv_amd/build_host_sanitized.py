"""Build librcattn_san.so: the same library with AddressSanitizer and
UndefinedBehaviorSanitizer on its host code (radix tree, planners, argument
checks, launch wrappers); the GPU code is built as usual.  For CPU test runs
only:

    python prefix_shared_kv_amd/build_host_sanitized.py
    LD_PRELOAD=$(/opt/rocm/llvm/bin/clang -print-file-name=libclang_rt.asan-x86_64.so) \\
    ASAN_OPTIONS=detect_leaks=0 RC_SANITIZED=1 python -m pytest tests -m "not gpu"

RC_SANITIZED=1 makes prefix_shared_kv_amd/_native.py load this library.  Every
file is compiled by clang (hipcc for the HIP sources, clang++ for the C++
ones) so that one sanitizer runtime serves all of them; the Python
interpreter is not instrumented, hence the preloaded runtime."""
from __future__ import annotations

import concurrent.futures as cf
import importlib.util
import os
import shutil
import subprocess

PKG = os.path.dirname(os.path.abspath(__file__))
_spec = importlib.util.spec_from_file_location("_rc_build", os.path.join(PKG, "build.py"))
B = importlib.util.module_from_spec(_spec)
_spec.loader.exec_module(B)

CLANGXX = "/opt/rocm/llvm/bin/clang++"
OUT = os.path.join(B.BUILD, "san")
LIB = os.path.join(PKG, "librcattn_san.so")
# host-side instrumentation only (the device pass is left as it is)
HOST_ONLY_SAN = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
                 "-Xarch_host", "-fno-omit-frame-pointer", "-Xarch_host", "-fno-sanitize-recover=undefined"]
CXX_SAN = ["-fsanitize=address,undefined", "-fno-omit-frame-pointer", "-fno-sanitize-recover=undefined"]


def build() -> str:
    os.makedirs(OUT, exist_ok=True)
    hip, cpp = B.sources()
    jobs = []
    for s in hip:
        o = os.path.join(OUT, os.path.basename(s) + ".o")
        jobs.append([B.HIPCC, *B.HIP_FLAGS, "-g", *HOST_ONLY_SAN, "-c", s, "-o", o])
    for s in cpp:
        o = os.path.join(OUT, os.path.basename(s) + ".o")
        jobs.append([CLANGXX, *B.CXX_FLAGS, "-g", *CXX_SAN, "-c", s, "-o", o])
    with cf.ThreadPoolExecutor(max_workers=8) as ex:
        list(ex.map(B._run, jobs))
    objs = [j[-1] for j in jobs]
    tmp = LIB + ".tmp"
    # the sanitizer runtime is not linked in: the process preloads it
    B._run([CLANGXX, "-shared", "-fPIC", "-pthread", *CXX_SAN, "-shared-libsan", "-o", tmp, *objs,
            "-L/opt/rocm/lib", "-lamdhip64", "-Wl,-rpath,/opt/rocm/lib"])
    shutil.move(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build())
