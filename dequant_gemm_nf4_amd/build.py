"""Build libbnbx.so (the HIP kernels and the C ABI of include/bnbx.h) for
gfx950, in-tree, with hipcc.  ``python -m dequant_gemm_nf4_amd.build``."""

from __future__ import annotations

import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libbnbx.so")
SOURCES = ["bnbx_api.hip", "bnbx_quant.hip", "bnbx_dequant.hip", "bnbx_gemv.hip", "bnbx_gemv16.hip",
           "bnbx_gemv_grouped.hip", "bnbx_gemv_lora.hip",
           "bnbx_gemm.hip",
           "bnbx_gemm_dx.hip", "bnbx_lora.hip", "bnbx_probe.hip"]

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = [
    "--offload-arch=gfx950",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-fvisibility=hidden",
    # every floating-point rounding step is spelled out in the source; the
    # compiler must not fuse a multiply and an add on its own
    "-ffp-contract=off",
    # no packed fp32 VALU forms
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", os.path.join(ROOT, "include"),
]


def _run(cmd):
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        sys.stderr.write(r.stdout + r.stderr)
        raise RuntimeError("hipcc failed: " + " ".join(cmd))
    return r


def build(verbose: bool = False) -> str:
    """Compile every source and link libbnbx.so; returns the library path."""
    os.makedirs(BUILD, exist_ok=True)
    objs = []
    procs = []
    for src in SOURCES:
        obj = os.path.join(BUILD, src.replace(".hip", ".o"))
        cmd = [HIPCC, *FLAGS, "-c", os.path.join(CSRC, src), "-o", obj]
        if verbose:
            print(" ".join(cmd))
        procs.append((cmd, subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.PIPE,
                                            text=True)))
        objs.append(obj)
    for cmd, p in procs:
        out, err = p.communicate()
        if p.returncode != 0:
            sys.stderr.write(out + err)
            raise RuntimeError("hipcc failed: " + " ".join(cmd))
    tmp = LIB + ".tmp"
    _run([HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", *objs, "-o", tmp])
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
