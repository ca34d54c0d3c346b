"""Build libq4.so (the HIP kernels and the C ABI) in-tree for gfx950.

    python int4_quantized_decode_q4_amd/build.py

This file is loaded by path, never through the package: importing the
package needs a built (and current) libq4.so, which is what this makes.

Each source is compiled by hipcc to an object under ``_build/`` (in
parallel), then linked into ``int4_quantized_decode_q4_amd/libq4.so``.
"""
from __future__ import annotations

import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(ROOT, "_build")
LIBRARY = os.path.join(PKG, "libq4.so")
SOURCES = ["q4_kernels.hip", "q4_gemm.hip", "q4_attention.hip", "q4_chain.hip", "q4_probe.hip",
           "q4_api.cpp"]
ARCH = "gfx950"

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
    # packed FP32 instructions are left to no one (see the build notes)
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-command-line-argument",
    f"-I{os.path.join(ROOT, 'include')}",
]


def sources_digest() -> str:
    """SHA-256 (first 16 hex digits) over the library's sources: every file
    of csrc/ and include/q4.h, in name order.  The build stamps it into the
    library (q4_source_hash), so a loaded library can be checked against the
    sources it claims to come from."""
    import hashlib
    h = hashlib.sha256()
    files = sorted(os.listdir(CSRC)) + ["../../include/q4.h"]
    for name in files:
        path = os.path.normpath(os.path.join(CSRC, name))
        if os.path.isfile(path):
            h.update(name.encode())
            with open(path, "rb") as f:
                h.update(f.read())
    return h.hexdigest()[:16]


def _compile(src: str, extra: list[str]) -> str:
    obj = os.path.join(BUILD, os.path.basename(src) + ".o")
    stamp = f'-DQ4_SOURCE_HASH="{sources_digest()}"'
    cmd = [HIPCC, *FLAGS, stamp, *extra, "-x", "hip", "-c", os.path.join(CSRC, src), "-o", obj]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{res.stdout}\n{res.stderr}")
    return obj


def build(extra: list[str] | None = None, out: str = LIBRARY) -> str:
    """Compile every HIP source for gfx950 and link libq4.so; returns its path."""
    extra = list(extra or [])
    os.makedirs(BUILD, exist_ok=True)
    with ThreadPoolExecutor(max_workers=len(SOURCES)) as ex:
        objs = list(ex.map(lambda s: _compile(s, extra), SOURCES))
    tmp = out + ".tmp%d" % os.getpid()
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"link failed:\n{res.stdout}\n{res.stderr}")
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    print(build(sys.argv[1:]))
