"""Build libgemvgemm.so from csrc/*.hip with hipcc for gfx950.

    python -m gemv_gemm_f32_amd.build [--save-temps DIR]

Each translation unit is compiled separately (no relocatable device code) and
linked into one shared library next to this file.  Packed fp32 VALU forms are
switched off in the device compiler (``-packed-fp32-ops``); the host pass
warns that it does not know that feature, which is harmless.
"""
from __future__ import annotations

import argparse
import glob
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libgemvgemm.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"

CFLAGS = [
    "--offload-arch=" + ARCH, "-O3", "-std=c++17", "-fPIC",
    "-mcode-object-version=5",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # the packed-weight GEMV multiplies binary16 subnormals: keep denormals
    "-fno-gpu-flush-denormals-to-zero",
    "-Wall", "-Wno-unused-command-line-argument",
]


def sources():
    return sorted(glob.glob(os.path.join(CSRC, "*.hip")))


def build(save_temps: str | None = None, verbose: bool = False) -> str:
    """Compile every kernel and the C entry points; returns the library path."""
    objdir = os.path.join(HERE, "_build")
    os.makedirs(objdir, exist_ok=True)
    objs = []
    for src in sources():
        obj = os.path.join(objdir, os.path.basename(src)[:-4] + ".o")
        cmd = [HIPCC] + CFLAGS + ["-c", src, "-o", obj]
        if save_temps:
            os.makedirs(save_temps, exist_ok=True)
            cmd += ["-save-temps=obj"]
            obj_t = os.path.join(save_temps, os.path.basename(obj))
            cmd[-1] = obj_t
            obj = obj_t
        if verbose:
            print(" ".join(cmd), flush=True)
        r = subprocess.run(cmd, capture_output=True, text=True)
        err = "\n".join(ln for ln in r.stderr.splitlines()
                        if "packed-fp32-ops" not in ln)
        if r.returncode != 0:
            raise RuntimeError("hipcc failed on %s:\n%s" % (src, err))
        if err.strip() and verbose:
            print(err, file=sys.stderr)
        objs.append(obj)
    tmp = LIB + ".tmp%d" % os.getpid()
    cmd = [HIPCC, "--offload-arch=" + ARCH, "-shared", "-fPIC", "-o", tmp] + objs
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("link failed:\n" + r.stderr)
    os.replace(tmp, LIB)
    return LIB


def build_probes(src: str, out: str) -> str:
    """Compile a stand-alone HIP source (the benchmark's probe kernels) into
    the shared library `out`, with the library's device flags."""
    tmp = out + ".tmp%d" % os.getpid()
    cmd = [HIPCC] + CFLAGS + ["-shared", src, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        err = "\n".join(ln for ln in r.stderr.splitlines() if "packed-fp32-ops" not in ln)
        raise RuntimeError("hipcc failed on %s:\n%s" % (src, err))
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    ap = argparse.ArgumentParser()
    ap.add_argument("--save-temps", default=None)
    ap.add_argument("-v", action="store_true")
    a = ap.parse_args()
    print(build(a.save_temps, a.v))
