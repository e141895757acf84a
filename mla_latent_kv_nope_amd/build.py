"""Build libmla.so (the HIP kernels + C ABI) in-tree for gfx950 with hipcc.

    python -m mla_latent_kv_nope_amd.build [--asm]

`--asm` also writes the device assembly of every kernel file next to the
object files under _build/ (used to check register use and instruction mix).
"""
from __future__ import annotations

import argparse
import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libmla.so")

SOURCES = ["mla_api.cpp", "k_append.hip", "k_absorb.hip", "k_decode.hip", "k_combine.hip", "noalloc.hip",
           "k_out_proj.hip", "k_project.hip",
           "k_prefill.hip"]
ARCH = "gfx950"
FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-fPIC", "-std=c++17", "-Wall",
    # code object v5 loads on every ROCm runtime a PyTorch wheel may bundle
    "-mcode-object-version=5",
    "-I", os.path.join(ROOT, "include"),
    # packed fp32 VALU ops are kept out of every kernel
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
]


def hipcc() -> str:
    p = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(p):
        raise RuntimeError("hipcc not found; ROCm is required to build libmla")
    return p


def _compile(src: str, asm: bool) -> str:
    obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
    cmd = [hipcc(), *FLAGS, "-c", os.path.join(CSRC, src), "-o", obj]
    if src.endswith(".hip"):
        cmd[1:1] = ["-x", "hip"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stderr}")
    if asm and src.endswith(".hip"):
        s_out = os.path.join(BUILD, os.path.splitext(src)[0] + f"-{ARCH}.s")
        cmd_s = [hipcc(), "-x", "hip", *FLAGS, "--cuda-device-only", "-S",
                 os.path.join(CSRC, src), "-o", s_out]
        r2 = subprocess.run(cmd_s, capture_output=True, text=True)
        if r2.returncode != 0:
            raise RuntimeError(f"hipcc -S failed for {src}:\n{r2.stderr}")
    return obj


def build(asm: bool = False, verbose: bool = True) -> str:
    os.makedirs(BUILD, exist_ok=True)
    with cf.ThreadPoolExecutor(max_workers=min(8, len(SOURCES))) as ex:
        objs = list(ex.map(lambda s: _compile(s, asm), SOURCES))
    tmp = LIB + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr}")
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB}")
    return LIB


if __name__ == "__main__":
    ap = argparse.ArgumentParser()
    ap.add_argument("--asm", action="store_true")
    args = ap.parse_args()
    try:
        build(asm=args.asm)
    except RuntimeError as e:
        print(e, file=sys.stderr)
        sys.exit(1)
