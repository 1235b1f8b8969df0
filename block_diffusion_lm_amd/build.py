"""Compile libbdattn.so (the HIP kernels and the C ABI) for gfx950, in-tree.

Usage: ``python -m block_diffusion_lm_amd.build`` (or ``build()`` from
Python).  Each source is compiled to an object with hipcc, in parallel, and
the objects are linked into ``block_diffusion_lm_amd/libbdattn.so``.
"""
from __future__ import annotations

import concurrent.futures
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(PKG, "csrc")
ROOT = os.path.dirname(PKG)
LIB = os.path.join(PKG, "libbdattn.so")
BUILD_DIR = os.path.join(ROOT, "_build")

SOURCES = ["api.cpp", "attn_fwd.hip", "attn_fwd_fp8.hip", "attn_bwd.hip"]

ARCH = "gfx950"

# Packed fp32 VALU instructions are disabled: plain scalar float code is
# used instead.
COMMON_FLAGS = [
    f"--offload-arch={ARCH}",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-Wall",
    "-Wno-unused-function",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", os.path.join(ROOT, "include"),
    "-I", CSRC,
]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build libbdattn.so)")


# Per-source code-generation options.
SOURCE_FLAGS = {}


def _compile(src: str, extra) -> str:
    obj = os.path.join(BUILD_DIR, os.path.basename(src) + ".o")
    extra = list(SOURCE_FLAGS.get(src, [])) + list(extra)
    cmd = [hipcc(), "-x", "hip", "-c", os.path.join(CSRC, src), "-o", obj] + COMMON_FLAGS + list(extra)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    return obj


def build(extra_flags=(), verbose: bool = True, out: str = None, source_flags=None) -> str:
    """Compile every source and link libbdattn.so (or ``out``); returns its path.

    ``source_flags`` maps a source file name to extra hipcc options for that
    file only (replacing SOURCE_FLAGS for the call)."""
    global BUILD_DIR
    lib_path = out or LIB
    if source_flags is not None:
        SOURCE_FLAGS.clear()
        SOURCE_FLAGS.update(source_flags)
    saved_dir = BUILD_DIR
    if out:
        BUILD_DIR = os.path.join(ROOT, "_build", os.path.basename(out) + ".d")
    os.makedirs(BUILD_DIR, exist_ok=True)
    with concurrent.futures.ThreadPoolExecutor(max_workers=len(SOURCES)) as ex:
        objs = list(ex.map(lambda s: _compile(s, extra_flags), SOURCES))
    BUILD_DIR = saved_dir
    tmp = lib_path + ".tmp"
    cmd = [hipcc(), "-shared", "-fPIC", f"--offload-arch={ARCH}", "-o", tmp] + objs
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, lib_path)
    if verbose:
        print(f"built {lib_path}")
    return lib_path


if __name__ == "__main__":
    # python -m block_diffusion_lm_amd.build [--out PATH] [hipcc options...]
    # e.g. --out _build/libbdattn_poison.so -DBDATTN_LDS_POISON for the LDS
    # poison debug build (load it with BDATTN_LIB=PATH)
    args = sys.argv[1:]
    out = None
    if "--out" in args:
        i = args.index("--out")
        out = os.path.abspath(args[i + 1])
        args = args[:i] + args[i + 2:]
    build(args, out=out)
