"""Build libbrq.so (the C-ABI library) for gfx950 with hipcc.

Usage: python -m binary_weight_gemm_amd.build  (or build() from Python).
Objects go to binary_weight_gemm_amd/_build/, the library next to this file.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
BUILD = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "libbrq.so")

SOURCES = ["abi.hip", "pack.hip", "dec.hip", "tile.hip", "pf.hip", "dbf.hip", "moe.hip", "kron.hip", "mid.hip", "lr.hip", "q8.hip", "noalloc.hip", "gsync.hip"]

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-Wall", "-Wno-unused-function",
    # no packed-fp32 instructions anywhere in the device code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", os.path.join(ROOT, "include"), "-I", CSRC,
]


#: per-source code generation options: the mid-size product keeps its
#: matrix-core results in ordinary vector registers (its group sums feed
#: vector FMAs; the accumulator-register form costs a move per result)
SOURCE_FLAGS = {"mid.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"]}


def _compile(src: str) -> str:
    obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
    cmd = [HIPCC, *FLAGS, *SOURCE_FLAGS.get(src, []), "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stderr}")
    errs = [l for l in r.stderr.splitlines() if "packed-fp32-ops" not in l and l.strip()]
    if errs:
        sys.stderr.write("\n".join(errs) + "\n")
    return obj


#: reference kernels of the benchmark (streaming read, matrix-core loop), a
#: library of their own that only bench.py loads
REF_SOURCES = ["refk.hip"]
REF_LIB = os.path.join(HERE, "libbrq_ref.so")


def _link(objs, out):
    tmp = out + ".tmp"
    cmd = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr}")
    shutil.move(tmp, out)


#: the host layer (argument checks, status and error text, per-device state)
#: built again with AddressSanitizer and UndefinedBehaviorSanitizer on its
#: host code only (device code is unchanged), linked with the other objects
#: into a library of its own that a CPU test loads with the sanitizer runtime
#: preloaded; never loaded by the product
SAN_SOURCES = ["abi.hip", "noalloc.hip", "gsync.hip"]
SAN_LIB = os.path.join(BUILD, "libbrq_hostsan.so")
SAN_FLAGS = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
             "-Xarch_host", "-fno-sanitize-recover=undefined", "-Xarch_host", "-fno-omit-frame-pointer"]


def sanitizer_runtime() -> str:
    """Path of the shared AddressSanitizer runtime of the compiler hipcc uses."""
    clang = os.path.join(os.path.dirname(os.path.realpath(HIPCC)), "..", "llvm", "bin", "clang++")
    r = subprocess.run([clang, "-print-file-name=libclang_rt.asan-x86_64.so"], capture_output=True, text=True)
    return r.stdout.strip()


def _compile_san(src: str) -> str:
    obj = os.path.join(BUILD, "san_" + os.path.splitext(src)[0] + ".o")
    cmd = [HIPCC, *FLAGS, *SOURCE_FLAGS.get(src, []), *SAN_FLAGS, "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc (host sanitizers) failed for {src}:\n{r.stderr}")
    return obj


def build(jobs: int = 8) -> str:
    os.makedirs(BUILD, exist_ok=True)
    with cf.ThreadPoolExecutor(max_workers=jobs) as ex:
        futs = [ex.submit(_compile, s) for s in SOURCES + REF_SOURCES]
        sans = [ex.submit(_compile_san, s) for s in SAN_SOURCES]
        objs = [f.result() for f in futs]
        san_objs = [f.result() for f in sans]
    _link(objs[:len(SOURCES)], LIB)
    _link(objs[len(SOURCES):], REF_LIB)
    plain = [o for o, s in zip(objs[:len(SOURCES)], SOURCES) if s not in SAN_SOURCES]
    tmp = SAN_LIB + ".tmp"
    cmd = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-Xarch_host", "-fsanitize=address",
           "-Xarch_host", "-fsanitize=undefined", "-Xarch_host", "-shared-libsan", "-o", tmp, *san_objs, *plain]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link (host sanitizers) failed:\n{r.stderr}")
    shutil.move(tmp, SAN_LIB)
    return LIB


if __name__ == "__main__":
    print(build())
