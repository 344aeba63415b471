"""Compile the k3huf HIP library for gfx950, in-tree.

Produces lossless_huffman_decoding_amd/_lib/libk3huf.so from csrc/ with hipcc
(decode kernels and ring drivers, GPU encoder, FP8 exponent decoder) and g++
(host table builds, header parsing, packers).
Always recompiles when called (the build check wants a real compile).
"""

from __future__ import annotations

import os
import subprocess

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
OUT_DIR = os.path.join(PKG, "_lib")
LIB = os.path.join(OUT_DIR, "libk3huf.so")
ARCH = "gfx950"

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
# packed fp32 instructions stay off for all device code. The atomic
# optimizer is off so that the decode kernel's work-ticket atomic (one lane,
# answer needed a whole work unit later) is not turned into a wave-wide
# reduction that waits for the answer at once.
HIP_FLAGS = ["--offload-arch=" + ARCH, "-O3", "-std=c++17", "-fPIC", "-Wall",
             "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
             "-mllvm", "-amdgpu-atomic-optimizer-strategy=None",
             "-I" + os.path.join(ROOT, "include")]
HOST_FLAGS = ["-O2", "-std=c++17", "-fPIC", "-Wall", "-Wextra", "-pthread",
              "-I" + os.path.join(ROOT, "include")]


def _run(cmd):
    subprocess.check_call(cmd)


def build(verbose: bool = False) -> str:
    os.makedirs(OUT_DIR, exist_ok=True)
    bdir = os.path.join(OUT_DIR, "_obj")
    os.makedirs(bdir, exist_ok=True)
    objs = []
    for name in ("k3huf_decode", "k3huf_encode", "e8huf_decode", "k3huf_stream"):
        o = os.path.join(bdir, name + ".o")
        _run([HIPCC, *HIP_FLAGS, "-c", os.path.join(CSRC, name + ".hip"), "-o", o])
        objs.append(o)
    for name in ("k3huf_host", "e8huf_host"):
        o = os.path.join(bdir, name + ".o")
        _run(["g++", *HOST_FLAGS, "-c", os.path.join(CSRC, name + ".cpp"), "-o", o])
        objs.append(o)
    tmp = LIB + ".tmp%d" % os.getpid()
    _run([HIPCC, "--offload-arch=" + ARCH, "-shared", "-fPIC", "-pthread", *objs, "-o", tmp])
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build())
