"""Build libnsg.so (gfx950 HIP kernels + host runtime + C ABI) in-tree.

    python -m newton_schulz_gram_amd.build        # or __graft_entry__.build()

The library is compiled for gfx950 only.  Packed-fp32 instructions are turned
off for the device code; the host pass prints a harmless warning about that
target feature.
"""
from __future__ import annotations

import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libnsg.so")

SOURCES = ["nsg_api.cpp", "nsg_kernels.hip", "nsg_select.hip", "nsg_muon.hip"]
# per-source flags: the Muon-step kernels round every fp32 operation on its own
# (hipcc's default contraction would fuse multiply-adds and ignore pragmas)
EXTRA = {"nsg_muon.hip": ["-ffp-contract=off"]}
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"


def build(verbose: bool = False) -> str:
    """Compile every source and link libnsg.so; returns the library path."""
    objdir = os.path.join(PKG, "_build")
    os.makedirs(objdir, exist_ok=True)
    common = [
        f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
        "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
        "-I", INCLUDE, "-I", CSRC,
        "-Wall", "-Wno-unused-function",
    ]
    objs = []
    for src in SOURCES:
        obj = os.path.join(objdir, src + ".o")
        cmd = [HIPCC, *common, *EXTRA.get(src, []), "-x", "hip", "-c", os.path.join(CSRC, src), "-o", obj]
        _run(cmd, verbose)
        objs.append(obj)
    tmp = LIB + ".tmp"
    _run([HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp], verbose)
    os.replace(tmp, LIB)
    return LIB


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    out = "\n".join(l for l in r.stdout.splitlines()
                    if "packed-fp32-ops" not in l)  # host-pass notice, harmless
    if r.returncode != 0:
        raise RuntimeError(f"build failed: {' '.join(cmd)}\n{out}")
    if verbose and out.strip():
        print(out, flush=True)


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
