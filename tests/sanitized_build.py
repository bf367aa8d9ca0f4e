"""Builds of the oracle and of the library with AddressSanitizer and
UndefinedBehaviorSanitizer on their host code, for the CPU tests in
test_sanitizers.py.  They land in ``_build_san/`` (not tracked), keyed by a
digest of the sources and flags, so a second run reuses them.

- The oracle: g++ with -fsanitize=address,undefined (loaded under gcc's
  ASan runtime).
- The library: hipcc with the sanitizers on the host side only (each
  ``-fsanitize=`` behind ``-Xarch_host``) and the device side at -O1; it is
  only loaded on the CPU, where no kernel runs (loaded under clang's ASan
  runtime).
"""
from __future__ import annotations

import concurrent.futures
import glob
import hashlib
import os
import shutil
import subprocess

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
OUT = os.path.join(ROOT, "_build_san")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

ORACLE_SRC = os.path.join(ROOT, "oracle", "spconv_oracle.cpp")
ORACLE_FLAGS = ["-O1", "-g", "-std=c++17", "-fopenmp", "-shared", "-fPIC", "-fno-omit-frame-pointer",
                "-fsanitize=address,undefined", "-fno-sanitize-recover=undefined"]

CSRC = os.path.join(ROOT, "submanifold_sparse_convolution_device_amd", "csrc")
LIB_FLAGS = ["-O1", "-g", "-std=c++17", "-fPIC", "--offload-arch=gfx950",
             "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops", "-fno-omit-frame-pointer",
             "-Xarch_host", "-fsanitize=address,undefined", "-Xarch_host", "-fno-sanitize-recover=undefined",
             "-Xarch_device", "-O1", "-I", os.path.join(ROOT, "include")]


def _digest(paths, flags):
    h = hashlib.sha256()
    for p in paths:
        with open(p, "rb") as f:
            h.update(f.read())
    h.update(" ".join(flags).encode())
    return h.hexdigest()[:16]


def gcc_asan_runtime() -> str:
    return subprocess.run(["gcc", "-print-file-name=libasan.so"], capture_output=True, text=True,
                          check=True).stdout.strip()


def clang_asan_runtime() -> str:
    hits = sorted(glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
    return hits[-1] if hits else ""


def build_oracle() -> str:
    key = _digest([ORACLE_SRC], ORACLE_FLAGS)
    out = os.path.join(OUT, f"liboracle_san_{key}.so")
    if not os.path.exists(out):
        os.makedirs(OUT, exist_ok=True)
        subprocess.run(["g++", *ORACLE_FLAGS, "-o", out + ".tmp", ORACLE_SRC], check=True)
        os.replace(out + ".tmp", out)
    return out


def build_library() -> str:
    import submanifold_sparse_convolution_device_amd.build as lib_build

    srcs = [os.path.join(CSRC, s) for s in lib_build.SOURCES]
    headers = sorted(glob.glob(os.path.join(CSRC, "*.h"))) + [os.path.join(ROOT, "include", "spconv.h")]
    key = _digest(srcs + headers, LIB_FLAGS)
    out = os.path.join(OUT, f"libspconv_san_{key}.so")
    if os.path.exists(out):
        return out
    objdir = os.path.join(OUT, f"obj_{key}")
    os.makedirs(objdir, exist_ok=True)

    def compile_one(src):
        name = os.path.basename(src)
        obj = os.path.join(objdir, os.path.splitext(name)[0] + ".o")
        extra = lib_build.EXTRA_FLAGS.get(name, [])
        r = subprocess.run([HIPCC, *LIB_FLAGS, *extra, "-c", src, "-o", obj], capture_output=True, text=True)
        if r.returncode != 0:
            raise RuntimeError(f"sanitized build of {name} failed:\n{r.stderr[-4000:]}")
        return obj

    with concurrent.futures.ThreadPoolExecutor(max_workers=min(8, len(srcs))) as ex:
        objs = list(ex.map(compile_one, srcs))
    subprocess.run([HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-Xarch_host", "-fsanitize=address,undefined",
                    "-o", out + ".tmp", *objs], check=True, capture_output=True)
    os.replace(out + ".tmp", out)
    shutil.rmtree(objdir, ignore_errors=True)
    return out
