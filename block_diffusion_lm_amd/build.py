"""Compile libbdattn.so (the HIP kernels and the C ABI) for gfx950, in-tree.

Usage: ``python -m block_diffusion_lm_amd.build`` (or ``build()`` from
Python).  Each source is compiled to an object with hipcc, in parallel, and
the objects are linked into ``block_diffusion_lm_amd/libbdattn.so``.
"""
from __future__ import annotations

import concurrent.futures
import json
import os
import re
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

# The compiler's per-kernel resource report (registers, scratch, occupancy)
# of the last default build, for the checks in tests/test_kernel_resources.py.
RESOURCES = os.path.join(ROOT, "_build", "kernel_resources.json")

_REMARK = re.compile(r"remark:\s+(Function Name|VGPRs|AGPRs|ScratchSize \[bytes/lane\]|Occupancy \[waves/SIMD\]|"
                     r"LDS Size \[bytes/block\]|VGPRs Spill|SGPRs Spill):\s+(\S+)")
_FIELDS = {"VGPRs": "vgprs", "AGPRs": "agprs", "ScratchSize [bytes/lane]": "scratch",
           "Occupancy [waves/SIMD]": "waves_per_simd", "LDS Size [bytes/block]": "lds",
           "VGPRs Spill": "vgpr_spill", "SGPRs Spill": "sgpr_spill"}


def kernel_key(mangled: str) -> str:
    """``bd::<name><args>`` from a mangled kernel symbol, e.g.
    ``fwd_kernel<128,32,4,2,0>`` (integer and bool template arguments)."""
    m = re.match(r"_ZN2bd(\d+)", mangled)
    if not m:
        return mangled
    i = m.end()
    name = mangled[i:i + int(m.group(1))]
    rest = mangled[i + int(m.group(1)):]
    args = re.findall(r"L[ib](-?\d+)E", rest) if rest.startswith("I") else []
    return f"{name}<{','.join(args)}>" if args else name


def parse_resources(text: str) -> dict:
    """Per kernel, the fields of the compiler's kernel-resource-usage remarks."""
    out, cur = {}, None
    for m in _REMARK.finditer(text):
        field, value = m.group(1), m.group(2)
        if field == "Function Name":
            cur = out.setdefault(kernel_key(value), {})
        elif cur is not None:
            cur[_FIELDS[field]] = int(value)
    return out


def _compile(src: str, extra) -> tuple:
    obj = os.path.join(BUILD_DIR, os.path.basename(src) + ".o")
    extra = list(SOURCE_FLAGS.get(src, [])) + list(extra)
    cmd = ([hipcc(), "-x", "hip", "-c", os.path.join(CSRC, src), "-o", obj] + COMMON_FLAGS + list(extra) +
           ["-Rpass-analysis=kernel-resource-usage"])
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    return obj, parse_resources(r.stderr)


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
        results = list(ex.map(lambda s: _compile(s, extra_flags), SOURCES))
    BUILD_DIR = saved_dir
    objs = [obj for obj, _ in results]
    if not out and not extra_flags and source_flags is None:
        resources = {}
        for _, res in results:
            resources.update(res)
        os.makedirs(os.path.dirname(RESOURCES), exist_ok=True)
        with open(RESOURCES, "w") as f:
            json.dump(resources, f, indent=1, sort_keys=True)
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
