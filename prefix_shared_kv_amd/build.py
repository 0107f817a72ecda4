"""Build librcattn.so in-tree: HIP kernels for gfx950 (hipcc) plus the host
radix tree and planners (g++).  Run ``python prefix_shared_kv_amd/build.py``
(by path: importing the package would load the library being rebuilt)."""
from __future__ import annotations

import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "librcattn.so")
# measured ceilings (streaming read, MFMA loop) for the roofline figures: a
# library of its own, not part of the attention library
CEIL_SRC = os.path.join(CSRC, "ceilings", "ceilings.hip")
CEIL_LIB = os.path.join(PKG, "libceilings.so")

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"

HIP_FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-Wall",
    # keep the compiler from forming packed fp32 vector ops
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # no kernel relies on NaN semantics (slots past a range are never read),
    # and without this every fmaxf of an MFMA result is preceded by a
    # canonicalising v_max_f32 x, x: 35 more VALU instructions per 64-key stage
    "-fno-honor-nans",
    "-I", INCLUDE, "-I", CSRC,
]
CXX_FLAGS = ["-O2", "-std=c++17", "-fPIC", "-pthread", "-Wall", "-Wextra", "-I", INCLUDE, "-I", CSRC]


def _run(cmd):
    p = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    out = "\n".join(l for l in p.stdout.splitlines() if "packed-fp32-ops" not in l)
    if p.returncode != 0:
        raise RuntimeError(f"build step failed ({p.returncode}): {' '.join(cmd)}\n{out}")
    return out


def sources():
    hip = sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC) if f.endswith(".hip"))
    cpp = sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC) if f.endswith(".cpp"))
    return hip, cpp


def build(verbose: bool = False, jobs: int = 8) -> str:
    os.makedirs(BUILD, exist_ok=True)
    hip, cpp = sources()
    jobs_list = []
    for s in hip:
        o = os.path.join(BUILD, os.path.basename(s) + ".o")
        jobs_list.append(([HIPCC, *HIP_FLAGS, "-c", s, "-o", o], o))
    for s in cpp:
        o = os.path.join(BUILD, os.path.basename(s) + ".o")
        jobs_list.append((["g++", *CXX_FLAGS, "-c", s, "-o", o], o))
    with cf.ThreadPoolExecutor(max_workers=jobs) as ex:
        outs = list(ex.map(lambda j: _run(j[0]), jobs_list))
    if verbose:
        for o in outs:
            if o.strip():
                print(o)
    tmp = LIB + ".tmp"
    _run([HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-pthread", "-o", tmp, *[o for _, o in jobs_list]])
    shutil.move(tmp, LIB)
    tmp = CEIL_LIB + ".tmp"
    _run([HIPCC, *HIP_FLAGS, "-shared", "-o", tmp, CEIL_SRC])
    shutil.move(tmp, CEIL_LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
