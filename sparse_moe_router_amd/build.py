"""Build the gfx950 libraries in-tree with hipcc.

    python -m sparse_moe_router_amd.build

produces ``sparse_moe_router_amd/libmoe_layer.so`` (the layer's C ABI and
kernels), ``synth/libsynth.so`` (the device twin of the seeded input
generator used by tests and the benchmark) and ``synth/libsynth_host.so``
(its host twin in C, built with gcc) and
``sparse_moe_router_amd/libmoe_peaks.so`` (the two measurement kernels of
``include/moe_peaks.h``: sustainable HBM read and bf16 MFMA rates).
"""
from __future__ import annotations

import concurrent.futures as cf
import glob
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PKG = os.path.join(ROOT, "sparse_moe_router_amd")
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(ROOT, "_build")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

ARCH = "gfx950"
# -packed-fp32-ops: no v_pk_{add,mul,fma}_f32 in device code.
CFLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-Wall", "-Wno-unused-function",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
]

LIB = os.path.join(PKG, "libmoe_layer.so")
SYNTH_LIB = os.path.join(ROOT, "synth", "libsynth.so")
SYNTH_HOST_LIB = os.path.join(ROOT, "synth", "libsynth_host.so")
PEAKS_LIB = os.path.join(PKG, "libmoe_peaks.so")


def _run(cmd):
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    # hipcc's host pass warns that it does not know the packed-fp32 feature; drop that line only
    out = "\n".join(l for l in r.stdout.splitlines() if "packed-fp32-ops" not in l)
    if r.returncode != 0:
        raise RuntimeError(f"command failed ({r.returncode}): {' '.join(cmd)}\n{out}")
    return out


def _compile(src, obj, extra=()):
    return _run([HIPCC, *CFLAGS, *extra, "-c", src, "-o", obj])


def _link(objs, out):
    tmp = out + ".tmp"
    _run([HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp])
    os.replace(tmp, out)


def build_layer(verbose=False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    srcs = sorted(glob.glob(os.path.join(CSRC, "*.hip")))
    inc = ["-I", os.path.join(ROOT, "include"), "-I", CSRC]
    objs = [os.path.join(BUILD, os.path.basename(s) + ".o") for s in srcs]
    with cf.ThreadPoolExecutor(max_workers=min(8, len(srcs))) as ex:
        logs = list(ex.map(lambda so: _compile(so[0], so[1], inc), zip(srcs, objs)))
    if verbose:
        for l in logs:
            if l.strip():
                print(l)
    _link(objs, LIB)
    return LIB


def build_synth() -> str:
    os.makedirs(BUILD, exist_ok=True)
    obj = os.path.join(BUILD, "synth_fill.o")
    _compile(os.path.join(ROOT, "synth", "csrc", "synth_fill.hip"), obj)
    _link([obj], SYNTH_LIB)
    return SYNTH_LIB


def build_synth_host() -> str:
    tmp = SYNTH_HOST_LIB + ".tmp"
    _run(["gcc", "-O3", "-fPIC", "-shared", "-ffp-contract=off", "-std=c11",
          os.path.join(ROOT, "synth", "csrc", "synth_host.c"), "-o", tmp])
    os.replace(tmp, SYNTH_HOST_LIB)
    return SYNTH_HOST_LIB


def build_peaks() -> str:
    os.makedirs(BUILD, exist_ok=True)
    obj = os.path.join(BUILD, "peaks.o")
    _compile(os.path.join(PKG, "peaks", "peaks.hip"), obj, ["-I", os.path.join(ROOT, "include")])
    _link([obj], PEAKS_LIB)
    return PEAKS_LIB


def build_all(verbose=False):
    return build_layer(verbose), build_synth(), build_synth_host(), build_peaks()


if __name__ == "__main__":
    for p in build_all(verbose="-v" in sys.argv):
        print("built", p)
