"""Build the gfx950 shared library in-tree with hipcc.

    python -m mla_absorbed_latent_amd.build        (or __graft_entry__.build())

Produces mla_absorbed_latent_amd/lib/libmla_absorbed_latent.so from the HIP
kernels and the C++ host layer.  Always recompiles (the build is a check too).
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(PKG, "csrc")
LIBDIR = os.path.join(PKG, "lib")
LIBNAME = "libmla_absorbed_latent.so"
OBJDIR = os.path.join(PKG, "_build")

ARCH = "gfx950"
COMMON = ["-O3", "-fPIC", "-std=c++17", "-Wall", "-Wno-unused-function"]
# Packed fp32 VALU instructions are disabled for all device code.
DEVICE = ["--offload-arch=" + ARCH, "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build the library)")


def sources():
    out = []
    for sub in ("kernels", "host"):
        d = os.path.join(CSRC, sub)
        for f in sorted(os.listdir(d)):
            if f.endswith((".hip", ".cpp")):
                out.append(os.path.join(d, f))
    return out


def _compile(src: str, cc: str) -> str:
    obj = os.path.join(OBJDIR, os.path.basename(src) + ".o")
    flags = COMMON + (DEVICE if src.endswith(".hip") else ["-D__HIP_PLATFORM_AMD__"])
    cmd = [cc] + flags + ["-c", src, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("compile failed: %s\n%s\n%s" % (" ".join(cmd), r.stdout, r.stderr))
    return obj


def build(verbose: bool = True) -> str:
    cc = hipcc()
    os.makedirs(OBJDIR, exist_ok=True)
    os.makedirs(LIBDIR, exist_ok=True)
    srcs = sources()
    with cf.ThreadPoolExecutor(max_workers=min(8, len(srcs))) as ex:
        objs = list(ex.map(lambda s: _compile(s, cc), srcs))
    out = os.path.join(LIBDIR, LIBNAME)
    tmp = out + ".tmp"
    cmd = [cc, "--offload-arch=" + ARCH, "-shared", "-fPIC", "-o", tmp] + objs
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("link failed: %s\n%s\n%s" % (" ".join(cmd), r.stdout, r.stderr))
    os.replace(tmp, out)
    if verbose:
        print("built", out, file=sys.stderr)
    return out


if __name__ == "__main__":
    build()
