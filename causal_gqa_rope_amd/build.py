"""Build libcgr.so in-tree for gfx950.

hipcc compiles every source under csrc/ to an object (in parallel); g++ links
the objects into causal_gqa_rope_amd/libcgr.so. The library is linked without
the HIP runtime: its HIP symbols resolve to the runtime already loaded in the
process (torch's, for the Python binding), so a process never carries two
HIP runtimes.

Run as ``python -m causal_gqa_rope_amd.build``.
"""

from __future__ import annotations

import concurrent.futures
import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD_DIR = os.path.join(HERE, "_build")
LIB_PATH = os.path.join(HERE, "libcgr.so")

SOURCES = [
    "cgr_api.hip",
    "rope_tables.hip",
    "varlen_sched.hip",
    "noalloc.hip",
    "attn_fwd_d32.hip",
    "attn_fwd_d64.hip",
    "attn_fwd_d128.hip",
    "attn_fwd_d256.hip",
    "attn_fp8.hip",
    "attn_bwd_d32.hip",
    "attn_bwd_d64.hip",
    "attn_bwd_d128.hip",
    "attn_decode_d32.hip",
    "attn_decode_d64.hip",
    "attn_decode_d128.hip",
    "qkv_d32.hip",
    "qkv_d64.hip",
    "qkv_d128.hip",
]

ARCH = os.environ.get("CGR_OFFLOAD_ARCH", "gfx950")


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (set HIPCC or install ROCm)")


def compile_flags() -> list:
    return [
        f"--offload-arch={ARCH}",
        "-O3",
        "-std=c++17",
        "-fPIC",
        "-fvisibility=hidden",
        # Keep the compiler from forming packed-f32 VALU instructions.
        "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
        "-I", INCLUDE,
        "-I", CSRC,
        "-Wno-unused-command-line-argument",
    ]


def _compile(src: str) -> str:
    obj = os.path.join(BUILD_DIR, os.path.splitext(src)[0] + ".o")
    cmd = [hipcc()] + compile_flags() + ["-c", os.path.join(CSRC, src), "-o", obj]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"compiling {src} failed:\n{' '.join(cmd)}\n{res.stdout}\n{res.stderr}")
    return obj


def build(jobs: int | None = None, verbose: bool = False) -> str:
    """Compile every source and link libcgr.so; returns the library path."""
    os.makedirs(BUILD_DIR, exist_ok=True)
    jobs = jobs or min(len(SOURCES), max(1, (os.cpu_count() or 2)))
    with concurrent.futures.ThreadPoolExecutor(max_workers=jobs) as ex:
        objs = list(ex.map(_compile, SOURCES))
    tmp = LIB_PATH + ".tmp"
    cmd = ["g++", "-shared", "-o", tmp] + objs + ["-Wl,-soname,libcgr.so", "-Wl,--no-undefined-version"]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"linking failed:\n{' '.join(cmd)}\n{res.stdout}\n{res.stderr}")
    os.replace(tmp, LIB_PATH)
    if verbose:
        print(f"built {LIB_PATH}")
    return LIB_PATH


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
