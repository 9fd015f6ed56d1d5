"""Builds libconvrot.so (hand-written HIP for gfx950) in-tree with hipcc.

Every translation unit is compiled for gfx950 only, with:
  -ffp-contract=off   no implicit a*b+c fusion: the fp32 steps of the method are exact
                      single-rounding operations, fused only where the source says fma;
  -Xclang -target-feature -Xclang -packed-fp32-ops
                      no packed fp32 instructions (hipcc's host pass warns that it does not
                      know the feature; that is harmless).
"""
import concurrent.futures as cf
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libconvrot.so")
# Measurement support for bench.py (memory ceilings of the rotate+quantize access pattern);
# a separate library, not part of libconvrot.so's ABI.
CEILING_SOURCE = "hbm_ceiling.hip"
CEILING_LIB = os.path.join(PKG, "libconvrot_ceiling.so")
BUILD = os.path.join(ROOT, "_build")
ARCH = "gfx950"

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = ["--offload-arch=" + ARCH, "-O3", "-std=c++17", "-fPIC", "-ffp-contract=off",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-Wall", "-Wno-unused-function", "-I", INCLUDE, "-I", CSRC]
SOURCES = ["rotate_quant.hip", "gemm_i8.hip", "gemm_rw.hip", "gemm_i8_wide.hip", "gemm_fp6.hip", "weight_quant.hip", "api.hip"]


def _compile(src: str) -> str:
    obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
    cmd = [HIPCC, *FLAGS, "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    err = "\n".join(l for l in r.stderr.splitlines() if "packed-fp32-ops" not in l)
    if r.returncode != 0:
        raise RuntimeError("hipcc failed for %s:\n%s" % (src, err))
    if err.strip():
        sys.stderr.write(err + "\n")
    return obj


def _link(objs, lib):
    tmp = lib + ".tmp%d" % os.getpid()
    r = subprocess.run([HIPCC, "--offload-arch=" + ARCH, "-shared", "-fPIC", *objs, "-o", tmp],
                       capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("link failed:\n" + r.stderr)
    os.replace(tmp, lib)


def build() -> str:
    """Compile every HIP source for gfx950, link libconvrot.so (and the bench's
    libconvrot_ceiling.so); returns the path of libconvrot.so."""
    os.makedirs(BUILD, exist_ok=True)
    with cf.ThreadPoolExecutor(max_workers=len(SOURCES) + 1) as ex:
        objs = list(ex.map(_compile, SOURCES + [CEILING_SOURCE]))
    _link(objs[:-1], LIB)
    _link(objs[-1:], CEILING_LIB)
    return LIB


if __name__ == "__main__":
    print(build())
