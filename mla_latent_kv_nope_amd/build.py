"""Build libmla.so (the HIP kernels + C ABI) in-tree for gfx950 with hipcc.

    python -m mla_latent_kv_nope_amd.build [--asm] [--sanitized]

`--asm` also writes the device assembly of every kernel file next to the
object files under _build/ (used to check register use and instruction mix).
`--sanitized` also builds _build/asan/libmla.so: the same kernels with the C
ABI layer (mla_api.cpp) compiled with AddressSanitizer and
UndefinedBehaviorSanitizer, for the host-only ABI tests (load it with the
sanitizer runtime preloaded; see tests/test_abi_sanitized.py).
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


# host-side sanitizers for the ABI layer (it has no device code)
SAN_FLAGS = ("-Xarch_host -fsanitize=address -Xarch_host -fsanitize=undefined "
             "-Xarch_host -fno-sanitize-recover=undefined -Xarch_host -fno-omit-frame-pointer").split()
SAN_LIB = os.path.join(BUILD, "asan", "libmla.so")


def sanitizer_runtime() -> str:
    """Path of clang's shared AddressSanitizer runtime (it also carries the
    UndefinedBehaviorSanitizer handlers), to be preloaded by the process that
    loads SAN_LIB."""
    r = subprocess.run([hipcc(), "-print-file-name=libclang_rt.asan-x86_64.so"], capture_output=True,
                       text=True)
    path = r.stdout.strip()
    if r.returncode != 0 or not os.path.isfile(path):
        raise RuntimeError("clang's libclang_rt.asan-x86_64.so not found")
    return path


def build_sanitized(verbose: bool = True) -> str:
    """SAN_LIB: the kernel objects of build() linked with a sanitized
    mla_api.o (the objects are rebuilt first unless each is newer than every
    source and header)."""
    newest = max(os.path.getmtime(os.path.join(CSRC, f)) for f in os.listdir(CSRC))
    objs_ok = all(os.path.exists(o) and os.path.getmtime(o) >= newest
                  for o in (os.path.join(BUILD, os.path.splitext(s)[0] + ".o") for s in SOURCES))
    if not objs_ok:
        build(verbose=False)
    san_dir = os.path.dirname(SAN_LIB)
    os.makedirs(san_dir, exist_ok=True)
    api_obj = os.path.join(san_dir, "mla_api.o")
    cmd = [hipcc(), *FLAGS, *SAN_FLAGS, "-c", os.path.join(CSRC, "mla_api.cpp"), "-o", api_obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for the sanitized mla_api.cpp:\n{r.stderr}")
    objs = [api_obj] + [os.path.join(BUILD, os.path.splitext(s)[0] + ".o") for s in SOURCES
                        if s != "mla_api.cpp"]
    tmp = SAN_LIB + ".tmp"
    r = subprocess.run([hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs],
                       capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr}")
    os.replace(tmp, SAN_LIB)
    if verbose:
        print(f"built {SAN_LIB}")
    return SAN_LIB


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
    ap.add_argument("--sanitized", action="store_true")
    args = ap.parse_args()
    try:
        build(asm=args.asm)
        if args.sanitized:
            build_sanitized()
    except RuntimeError as e:
        print(e, file=sys.stderr)
        sys.exit(1)
