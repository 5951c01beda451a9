"""Build libq4.so in-tree with hipcc for gfx950.

    python -m gemv_q4_affine_amd.build

Each source is compiled to an object in _build/ (in parallel), then linked
into gemv_q4_affine_amd/libq4.so.  Always recompiles: a build is the check
that every kernel still compiles for gfx950.
"""
from __future__ import annotations

import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libq4.so")

SOURCES = ["quant.hip", "gemv.hip", "gemm.hip", "gemm_big.hip", "gemm_q8.hip", "affine8.hip", "noalloc.hip",
           "capi.cpp"]

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

# Per-source flags.  The decode GEMVs are launch-latency bound: their leading
# scalar and pointer arguments (what a one-matrix launch reads) are preloaded
# into SGPRs at wave launch instead of being fetched from the argument block.
SOURCE_FLAGS = {"gemv.hip": ["-mllvm", "-amdgpu-kernarg-preload-count=16"]}

FLAGS = [
    "--offload-arch=gfx950",
    "-O3",
    "-fPIC",
    "-std=c++17",
    # quantiser codes are defined by separate binary32 multiply and add
    "-ffp-contract=off",
    # keep the compiler from emitting packed fp32 VALU ops
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-unused-command-line-argument",
    # gemm_big.hip names m0 among its copy instruction's clobbers on purpose
    "-Wno-inline-asm",
    "-I", INCLUDE,
    "-I", CSRC,
]


def _compile(src: str) -> str:
    obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
    cmd = [HIPCC, *FLAGS, *SOURCE_FLAGS.get(src, []), "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stdout}\n{r.stderr}")
    return obj


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    with ThreadPoolExecutor(max_workers=min(8, len(SOURCES))) as ex:
        objs = list(ex.map(_compile, SOURCES))
    tmp = LIB + ".tmp"
    cmd = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, LIB)
    _write_build_info()
    if verbose:
        print(f"built {LIB}")
    return LIB


BUILD_INFO = os.path.join(os.path.dirname(LIB), "build_info.json")


def _write_build_info() -> None:
    """Record the git commit the library was built from (and whether the tree
    differed from it) beside the library: copies of the tree without git
    metadata still name their source."""
    import json
    info = {"git_commit": None, "tree_modified": None}
    try:
        root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
        head = subprocess.run(["git", "-C", root, "rev-parse", "HEAD"], capture_output=True, text=True, timeout=10)
        if head.returncode == 0:
            info["git_commit"] = head.stdout.strip()
            st = subprocess.run(["git", "-C", root, "status", "--porcelain", "--untracked-files=no"],
                                capture_output=True, text=True, timeout=10)
            info["tree_modified"] = bool(st.stdout.strip()) if st.returncode == 0 else None
    except (OSError, subprocess.SubprocessError):
        pass
    with open(BUILD_INFO, "w") as f:
        json.dump(info, f)


# ---- host-side AddressSanitizer / UndefinedBehaviorSanitizer build -------------
# The host half of each source (argument checks, dispatch, size arithmetic,
# launch set-up) is instrumented; the device code is built plainly (at -O1:
# this build serves tests that make no GPU call, tests/test_abi_host.py).
# Load it into a process that preloads SAN_RUNTIME, with Q4_LIB_PATH
# pointing at it.
SAN_DIR = os.path.join(BUILD, "san")
SAN_LIB = os.path.join(SAN_DIR, "libq4_host_san.so")
SAN_RUNTIME = "/opt/rocm/llvm/lib/clang/22/lib/linux/libclang_rt.asan-x86_64.so"
SAN_FLAGS = [
    "--offload-arch=gfx950",
    "-O1", "-g", "-fPIC", "-std=c++17", "-fno-omit-frame-pointer",
    "-Xarch_host", "-fsanitize=address",
    "-Xarch_host", "-fsanitize=undefined",
    "-Xarch_host", "-fno-sanitize-recover=all",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-unused-command-line-argument", "-Wno-inline-asm", "-Wno-unused-result",
    "-I", INCLUDE, "-I", CSRC,
]


def _compile_san(src: str) -> str:
    obj = os.path.join(SAN_DIR, os.path.splitext(src)[0] + ".o")
    cmd = [HIPCC, *SAN_FLAGS, "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc (host, sanitized) failed for {src}:\n{r.stdout}\n{r.stderr}")
    return obj


def build_host_sanitized(verbose: bool = False) -> str:
    """Build SAN_LIB if any source is newer than it; return its path."""
    srcs = [os.path.join(CSRC, f) for f in os.listdir(CSRC)] + [os.path.join(INCLUDE, "q4.h")]
    if os.path.exists(SAN_LIB) and os.path.getmtime(SAN_LIB) >= max(os.path.getmtime(f) for f in srcs):
        return SAN_LIB
    os.makedirs(SAN_DIR, exist_ok=True)
    with ThreadPoolExecutor(max_workers=min(6, len(SOURCES))) as ex:
        objs = list(ex.map(_compile_san, SOURCES))
    tmp = SAN_LIB + ".tmp"
    cmd = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-Xarch_host", "-fsanitize=address",
           "-Xarch_host", "-fsanitize=undefined", "-shared-libsan", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link (sanitized) failed:\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, SAN_LIB)
    if verbose:
        print(f"built {SAN_LIB}")
    return SAN_LIB


if __name__ == "__main__":
    if "--host-sanitized" in sys.argv[1:]:
        build_host_sanitized(verbose=True)
    else:
        build(verbose=True)
    sys.exit(0)
