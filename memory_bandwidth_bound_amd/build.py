"""Build libkie.so (gfx950) in-tree.

    python -m memory_bandwidth_bound_amd.build

Host-only preparation code (kie_host.cpp) is compiled with g++; the kernels and
the C ABI with hipcc for gfx950. Object files go to _build/ at the repository
root; the shared library is written next to this file.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libkie.so")

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
GXX = os.environ.get("CXX", "g++")
ARCH = "gfx950"

HIP_FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
    # packed fp32 arithmetic stays off: hipcc -O3 must not emit v_pk_*_f32
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-unused-result",
]
CXX_FLAGS = ["-O2", "-std=c++17", "-fPIC", "-Wall"]


def _run(cmd):
    p = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    out = "\n".join(l for l in p.stdout.splitlines()
                    if "packed-fp32-ops" not in l and "is not a recognized feature" not in l)
    if p.returncode != 0:
        raise RuntimeError("build failed:\n" + " ".join(cmd) + "\n" + out)
    return out


def build(verbose: bool = False, defines=(), out: str = LIB, build_dir: str = BUILD) -> str:
    """Compile every source and link libkie.so; returns its path.

    defines: extra -D flags (kernel tuning knobs such as KIE_NB=6); out and
    build_dir place the library and objects elsewhere (for such variants)."""
    if not os.path.exists(HIPCC) and shutil.which("hipcc") is None:
        raise RuntimeError("hipcc not found")
    os.makedirs(build_dir, exist_ok=True)
    inc = ["-I", os.path.join(ROOT, "include"), "-I", CSRC]
    units = ["kie_decode", "kie_prefill", "kie_probes", "kie_api"]
    dflags = ["-D" + d for d in defines]
    jobs = [[GXX, *CXX_FLAGS, *dflags, *inc, "-c", os.path.join(CSRC, "kie_host.cpp"), "-o",
             os.path.join(build_dir, "kie_host.o")]]
    for u in units:
        jobs.append([HIPCC, *HIP_FLAGS, *dflags, *inc, "-c", os.path.join(CSRC, u + ".hip"), "-o",
                     os.path.join(build_dir, u + ".o")])
    with ThreadPoolExecutor(len(jobs)) as ex:
        outs = list(ex.map(_run, jobs))
    tmp = out + ".tmp"
    objs = [os.path.join(build_dir, n + ".o") for n in ["kie_host", *units]]
    outs.append(_run([HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]))
    os.replace(tmp, out)
    if verbose:
        for o in outs:
            if o.strip():
                print(o)
    return out


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
