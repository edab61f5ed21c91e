"""Build the HIP library ``libpa.so`` in-tree for gfx950.

Every source is compiled with hipcc for gfx950 only, with packed-fp32 VALU
instructions disabled, then linked into one shared library next to this
file. The SHA-256 of the sources (``srchash.source_sha256``) is written to a
generated header in the build folder and baked into ``pa_version()``. Run as
``python -m paged_kv_cache_66_amd.build``.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

if __package__ in (None, ""):
    sys.path.insert(0, os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
    from paged_kv_cache_66_amd.srchash import source_sha256
else:
    from .srchash import source_sha256

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(os.path.dirname(HERE), "include")
BUILD_DIR = os.path.join(HERE, "_build")
LIB_PATH = os.path.join(HERE, "libpa.so")
SOURCES = ["pa_api.cpp", "store_kvcache.hip", "decode.hip", "prefill.hip"]
ARCH = "gfx950"


def hipcc() -> str:
    root = os.environ.get("ROCM_PATH", "/opt/rocm")
    cand = os.path.join(root, "bin", "hipcc")
    return cand if os.path.exists(cand) else (shutil.which("hipcc") or "hipcc")


COMMON_FLAGS = [
    f"--offload-arch={ARCH}",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-Wall",
    "-Wno-unused-function",
    # packed fp32 VALU forms stay out of every kernel
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
]


def _compile(src: str) -> str:
    obj = os.path.join(BUILD_DIR, os.path.splitext(src)[0] + ".o")
    cmd = [hipcc(), *COMMON_FLAGS, "-I", CSRC, "-I", INCLUDE, "-I", BUILD_DIR, "-c",
           os.path.join(CSRC, src), "-o", obj]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{' '.join(cmd)}\n{res.stdout}\n{res.stderr}")
    return obj


def build(verbose: bool = False) -> str:
    """Compile all sources and link ``libpa.so``; returns its path."""
    os.makedirs(BUILD_DIR, exist_ok=True)
    digest = source_sha256()
    with open(os.path.join(BUILD_DIR, "pa_srchash.h"), "w") as f:
        f.write(f'#define PA_SOURCE_SHA256 "{digest}"\n')
    with ThreadPoolExecutor(max_workers=min(len(SOURCES), os.cpu_count() or 1)) as ex:
        objs = list(ex.map(_compile, SOURCES))
    tmp = LIB_PATH + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"link failed:\n{' '.join(cmd)}\n{res.stdout}\n{res.stderr}")
    os.replace(tmp, LIB_PATH)
    if verbose:
        print(f"built {LIB_PATH} (src-sha256:{digest})")
    return LIB_PATH


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
