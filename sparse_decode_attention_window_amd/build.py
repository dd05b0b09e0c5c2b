"""Build libkvsel.so for gfx950 in-tree.

hipcc compiles every .hip source (device code for gfx950 only); the host-only
budget helper is compiled with g++ and -ffp-contract=off.  Objects go to
_build/ next to this file; the shared library lands in the package directory.
Usage: python -m sparse_decode_attention_window_amd.build  (or build())
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
BUILD = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libkvsel.so")
PROBE_SRC = os.path.join(PKG, "probe", "hbm_probe.hip")
PROBE_LIB = os.path.join(PKG, "libkvsel_probe.so")   # the benchmark's HBM stream, not the method
ARCH = "gfx950"

HIPCC = os.environ.get("HIPCC", shutil.which("hipcc") or "/opt/rocm/bin/hipcc")
HIP_FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-Wall",
    "-Wno-unused-variable", "-Wno-unused-function",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # matrix-core results straight into VGPRs: the softmax code reads every
    # accumulator element, and AGPR results would cost one move per element
    "-mllvm", "-amdgpu-mfma-vgpr-form",
    "-I" + os.path.join(ROOT, "include"),
]
CXX_FLAGS = ["-O2", "-std=c++17", "-fPIC", "-ffp-contract=off", "-D__HIP_PLATFORM_AMD__",
             "-I/opt/rocm/include", "-I" + os.path.join(ROOT, "include")]


def _run(cmd):
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    out = "\n".join(l for l in r.stdout.splitlines() if "packed-fp32-ops" not in l)
    if r.returncode != 0:
        raise RuntimeError(f"command failed ({r.returncode}): {' '.join(cmd)}\n{out}")
    return out


def build(verbose: bool = False, out: str = LIB, build_dir: str = BUILD,
          defines: tuple = ()) -> str:
    """Compile every source and link `out`; `defines` are extra -D flags."""
    os.makedirs(build_dir, exist_ok=True)
    jobs = []
    for f in sorted(os.listdir(CSRC)):
        src = os.path.join(CSRC, f)
        obj = os.path.join(build_dir, f + ".o")
        if f.endswith(".hip"):
            jobs.append([HIPCC, *HIP_FLAGS, *[f"-D{d}" for d in defines], "-c", src, "-o", obj])
        elif f.endswith(".cpp"):
            jobs.append(["g++", *CXX_FLAGS, "-c", src, "-o", obj])
    with ThreadPoolExecutor(min(8, len(jobs))) as ex:
        outs = list(ex.map(_run, jobs))
    if verbose:
        for o in outs:
            if o.strip():
                print(o)
    objs = [j[-1] for j in jobs]
    tmp = out + ".tmp"
    _run([HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs])
    os.replace(tmp, out)
    return out


def build_probe(out: str = PROBE_LIB) -> str:
    """The benchmark's HBM stream probe, a library of its own."""
    tmp = out + ".tmp"
    _run([HIPCC, *HIP_FLAGS, "-shared", PROBE_SRC, "-o", tmp])
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
    print(build_probe())
