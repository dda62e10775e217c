"""Compiles the HIP library ``libinvariant_moe.so`` for gfx950 in-tree.

Flags: -O3; fp contraction off (every fused multiply-add in the kernels is
written explicitly, so the arithmetic is the source's on every path); IEEE
fp32 division; denormals kept; packed-fp32 instructions disabled.
"""
from __future__ import annotations

import hashlib
import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(PKG, "_build_obj")
LIB = os.path.join(PKG, "libinvariant_moe.so")

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"

DEVICE_FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
    "-ffp-contract=off", "-fhip-fp32-correctly-rounded-divide-sqrt",
    "-fno-gpu-flush-denormals-to-zero",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-result",
]
SOURCES = ["router.hip", "permute.hip", "gemm.hip", "combine.hip", "quant.hip", "noalloc.hip",
           "fused.hip",
           "abi.cpp"]
HEADER = os.path.join(os.path.dirname(PKG), "include", "moe.h")


def source_hash() -> str:
    """Hash of everything the library is built from: the kernel and host
    sources, the public header and these build flags.  The build compiles it
    into the library (moe_build_id), so a loaded binary can be checked
    against the sources next to it."""
    h = hashlib.sha256()
    files = sorted(f for f in os.listdir(CSRC) if f.endswith((".hip", ".hpp", ".cpp")))
    for name in files + ["moe.h"]:
        path = HEADER if name == "moe.h" else os.path.join(CSRC, name)
        h.update(name.encode() + b"\0")
        with open(path, "rb") as f:
            h.update(f.read())
    h.update(" ".join(DEVICE_FLAGS + SOURCES).encode())
    return h.hexdigest()[:16]


def _compile(src: str, build_id: str) -> str:
    obj = os.path.join(BUILD, src + ".o")
    cmd = [HIPCC, *DEVICE_FLAGS, f'-DMOE_BUILD_ID="{build_id}"', "-c", os.path.join(CSRC, src),
           "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    err = "\n".join(ln for ln in (r.stdout + r.stderr).splitlines()
                    if "packed-fp32-ops" not in ln)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{err}")
    if err.strip():
        sys.stderr.write(err + "\n")
    return obj


def build_library() -> str:
    os.makedirs(BUILD, exist_ok=True)
    build_id = source_hash()
    with ThreadPoolExecutor(max_workers=min(8, len(SOURCES))) as ex:
        objs = list(ex.map(lambda src: _compile(src, build_id), SOURCES))
    tmp = LIB + ".tmp"
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("link failed:\n" + r.stdout + r.stderr)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build_library())
