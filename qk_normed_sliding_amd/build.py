"""Build libsa_attn.so (HIP kernels + C ABI) in-tree for gfx950 with hipcc.

Usage: python qk_normed_sliding_amd/build.py   (always recompiles; run it as a
file: importing the package loads the library, which must exist first)
"""

from __future__ import annotations

import concurrent.futures as cf
import glob
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libsa_attn.so")
ARCH = "gfx950"

# Packed fp32 VALU forms are kept out of the generated code on purpose.
DEVICE_FLAGS = ["-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]
COMMON = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}", "-fvisibility=hidden",
          "-I", os.path.join(ROOT, "include"), "-I", CSRC, "-Wall", "-Wno-unused-function"]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build libsa_attn.so)")


def _run(cmd):
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    # hipcc's host pass does not know the packed-fp32 feature; that warning is harmless
    out = "\n".join(ln for ln in r.stdout.splitlines() if "packed-fp32-ops" not in ln)
    if r.returncode != 0:
        raise RuntimeError(f"command failed ({r.returncode}): {' '.join(cmd)}\n{out}")
    return out


def build(verbose: bool = False) -> str:
    cc = hipcc()
    os.makedirs(BUILD, exist_ok=True)
    srcs = sorted(glob.glob(os.path.join(CSRC, "*.hip")))
    objs = [os.path.join(BUILD, os.path.basename(s)[:-4] + ".o") for s in srcs]
    jobs = max(1, min(len(srcs), int(os.environ.get("MAX_JOBS", os.cpu_count() or 4))))
    with cf.ThreadPoolExecutor(jobs) as ex:
        outs = list(ex.map(lambda so: _run([cc, *COMMON, *DEVICE_FLAGS, "-c", so[0], "-o", so[1]]),
                           zip(srcs, objs)))
    tmp = LIB + ".tmp"
    outs.append(_run([cc, "-shared", "-fPIC", f"--offload-arch={ARCH}", *objs, "-o", tmp]))
    os.replace(tmp, LIB)
    if verbose:
        for o in outs:
            if o.strip():
                print(o)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
