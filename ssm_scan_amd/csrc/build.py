"""Build libloglin.so for gfx950 with hipcc (in-tree, no JIT cache).

Compiles the host C-ABI unit, the decode and gated DeltaNet units, six forward instantiation
units (io type x chunk) and five backward ones in parallel, then links
ssm_scan_amd/_lib/libloglin.so.

build_host_asan() links a second copy, _build/asan/libloglin.so, whose host
code (the C-ABI layer: argument checks, workspace plans, launch sequences) is
built with AddressSanitizer; device code is the same.  The ABI tests run
against it on the CPU with the sanitizer runtime preloaded (asan_runtime()).
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
PKG = os.path.dirname(HERE)
ROOT = os.path.dirname(PKG)
INCLUDE = os.path.join(ROOT, "include")
OUT_DIR = os.path.join(PKG, "_lib")
BUILD_DIR = os.path.join(ROOT, "_build")
LIB = os.path.join(OUT_DIR, "libloglin.so")

ARCH = "gfx950"
HIPCC = os.environ.get("HIPCC") or shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
    # never emit packed fp32 ops (v_pk_*_f32)
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", INCLUDE, "-I", HERE,
]


def _units():
    units = [("loglin_host", os.path.join(HERE, "loglin_host.cpp"), []),
             ("loglin_decode", os.path.join(HERE, "loglin_decode.hip"), []),
             ("loglin_gdn", os.path.join(HERE, "loglin_gdn.hip"), []),
             ("loglin_noalloc", os.path.join(HERE, "loglin_noalloc.hip"), [])]
    for io in ("bf16", "f32"):
        for chunk in (16, 32, 64):
            units.append((f"loglin_inst_{io}_{chunk}",
                          os.path.join(HERE, "loglin_inst.hip"),
                          [f"-DLOGLIN_IO={io}", f"-DLOGLIN_CHUNK={chunk}"]))
    for io, chunks in (("bf16", (32, 64)), ("f32", (16, 32, 64))):
        for chunk in chunks:
            units.append((f"loglin_bwd_{io}_{chunk}",
                          os.path.join(HERE, "loglin_bwd_inst.hip"),
                          [f"-DLOGLIN_IO={io}", f"-DLOGLIN_CHUNK={chunk}"]))
    return units


def _compile(unit):
    name, src, defs = unit
    obj = os.path.join(BUILD_DIR, name + ".o")
    lang = ["-x", "hip"] if src.endswith(".cpp") else []
    cmd = [HIPCC, *FLAGS, *defs, *lang, "-c", src, "-o", obj]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"compile failed: {' '.join(cmd)}\n{res.stdout}\n{res.stderr}")
    return obj


def build(jobs: int | None = None, verbose: bool = False) -> str:
    os.makedirs(BUILD_DIR, exist_ok=True)
    os.makedirs(OUT_DIR, exist_ok=True)
    jobs = jobs or min(8, os.cpu_count() or 1)
    with cf.ThreadPoolExecutor(jobs) as ex:
        objs = list(ex.map(_compile, _units()))
    tmp = LIB + ".tmp"
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"link failed: {' '.join(cmd)}\n{res.stdout}\n{res.stderr}")
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB}")
    return LIB


ASAN_DIR = os.path.join(BUILD_DIR, "asan")
ASAN_LIB = os.path.join(ASAN_DIR, "libloglin.so")
# host-side sanitizer only: each -fsanitize applies to the host pass
ASAN_FLAGS = ["-O1", "-g", "-Xarch_host", "-fsanitize=address",
              "-Xarch_host", "-fno-omit-frame-pointer"]
ASAN_LINK = ["-Xarch_host", "-fsanitize=address"]
ASAN_UNITS = ("loglin_host", "loglin_noalloc")


def asan_runtime() -> str:
    """Path of the compiler's AddressSanitizer runtime (to preload)."""
    clang = os.path.join(os.path.dirname(os.path.realpath(HIPCC)), "..", "llvm", "bin", "clang")
    if not os.path.exists(clang):
        clang = "/opt/rocm/llvm/bin/clang"
    res = subprocess.run([clang, "-print-file-name=libclang_rt.asan-x86_64.so"],
                         capture_output=True, text=True, check=True)
    return res.stdout.strip()


def build_host_asan(verbose: bool = False) -> str:
    """Link _build/asan/libloglin.so: the host units rebuilt with
    AddressSanitizer, every other object as built by build()."""
    os.makedirs(ASAN_DIR, exist_ok=True)
    units = {u[0]: u for u in _units()}
    objs = []
    for name, src, defs in units.values():
        if name in ASAN_UNITS:
            obj = os.path.join(ASAN_DIR, name + ".o")
            lang = ["-x", "hip"] if src.endswith(".cpp") else []
            flags = [f for f in FLAGS if f != "-O3"]
            cmd = [HIPCC, *flags, *ASAN_FLAGS, *defs, *lang, "-c", src, "-o", obj]
            res = subprocess.run(cmd, capture_output=True, text=True)
            if res.returncode != 0:
                raise RuntimeError(f"compile failed: {' '.join(cmd)}\n{res.stdout}\n{res.stderr}")
        else:
            obj = os.path.join(BUILD_DIR, name + ".o")
            if not os.path.exists(obj):
                obj = _compile((name, src, defs))
        objs.append(obj)
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", *ASAN_LINK, "-o", ASAN_LIB, *objs]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"link failed: {' '.join(cmd)}\n{res.stdout}\n{res.stderr}")
    if verbose:
        print(f"built {ASAN_LIB}")
    return ASAN_LIB


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
