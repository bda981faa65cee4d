"""Build libquest.so (gfx950 only) in-tree with hipcc.

    python query_aware_kv_amd/build.py          # or __graft_entry__.build()

Objects go to query_aware_kv_amd/_build/, the library to
query_aware_kv_amd/libquest.so.  Every call compiles from scratch.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libquest.so")
ARCH = "gfx950"

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

COMMON_FLAGS = [
    "-O3", "-std=c++17", "-fPIC", "-fvisibility=hidden",
    f"--offload-arch={ARCH}",
    # no packed-fp32 instructions in any generated code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function",
    f"-I{INCLUDE}", f"-I{CSRC}",
]

SOURCES = ["api.cpp", "meta.hip", "estimate.hip", "topk.hip", "attention.hip",
           "topk_attn.hip", "step.hip", "probe.hip",
           "union.hip"]


# Host-side AddressSanitizer + UndefinedBehaviorSanitizer for the CPU-only
# build the ABI tests run against (device code is built as usual).
SANITIZE_HOST = ("-Xarch_host -fsanitize=address -Xarch_host -fsanitize=undefined "
                 "-Xarch_host -fno-omit-frame-pointer -Xarch_host -g").split()
BUILD_SAN = os.path.join(PKG, "_build_san")
LIB_SAN = os.path.join(BUILD_SAN, "libquest_san.so")


def _compile(src: str, build_dir: str = BUILD, extra=()) -> str:
    obj = os.path.join(build_dir, os.path.basename(src) + ".o")
    cmd = [HIPCC, *COMMON_FLAGS, *extra, "-x", "hip", "-c", os.path.join(CSRC, src),
           "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{' '.join(cmd)}\n"
                           f"{r.stdout}\n{r.stderr}")
    return obj


def build(verbose: bool = False) -> str:
    if os.path.isdir(BUILD):
        shutil.rmtree(BUILD)
    os.makedirs(BUILD)
    with cf.ThreadPoolExecutor(max_workers=min(8, len(SOURCES))) as ex:
        objs = list(ex.map(_compile, SOURCES))
    tmp = LIB + ".tmp"
    cmd = [HIPCC, "-shared", "-fPIC", f"--offload-arch={ARCH}", *objs,
           "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB}")
    return LIB


def build_sanitized(verbose: bool = False) -> str:
    """libquest_san.so: the same sources with host code under ASan + UBSan
    (load it with the sanitizer runtime preloaded, QUEST_LIB pointing at
    it).  For the host-side ABI tests only: no kernel is launched there."""
    if os.path.isdir(BUILD_SAN):
        shutil.rmtree(BUILD_SAN)
    os.makedirs(BUILD_SAN)
    with cf.ThreadPoolExecutor(max_workers=min(8, len(SOURCES))) as ex:
        objs = list(ex.map(lambda s_: _compile(s_, BUILD_SAN, SANITIZE_HOST), SOURCES))
    cmd = [HIPCC, "-shared", "-fPIC", f"--offload-arch={ARCH}", *SANITIZE_HOST,
           "-shared-libsan", *objs, "-o", LIB_SAN]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    if verbose:
        print(f"built {LIB_SAN}")
    return LIB_SAN


def sanitizer_runtime() -> str:
    """The shared ASan runtime of hipcc's clang (to preload)."""
    clang = os.path.join(os.path.dirname(os.path.realpath(HIPCC)), "..", "llvm", "bin",
                         "clang")
    r = subprocess.run([clang, "-print-file-name=libclang_rt.asan-x86_64.so"],
                       capture_output=True, text=True)
    return r.stdout.strip()


if __name__ == "__main__":
    if "--sanitized" in sys.argv:
        build_sanitized(verbose=True)
    else:
        build(verbose=True)
    sys.exit(0)
