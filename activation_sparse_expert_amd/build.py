"""Build libmoeffn.so (hipcc, gfx950) in-tree."""
from __future__ import annotations

import hashlib
import os
import subprocess
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
OUT = os.path.join(HERE, "libmoeffn.so")
BUILD = os.path.join(HERE, "_build")

SOURCES = ["api.cpp", "expert_sparse_f16.hip", "expert_sparse_bf16.hip", "reduce.hip", "route.hip",
           "pack.hip", "dense_mfma.hip", "dense_gemm.hip", "calibrate.hip",
           "eamc.hip", "expert_sparse_bits.hip"]

HEADER = os.path.join(os.path.dirname(HERE), "include", "moeffn.h")

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = [
    "--offload-arch=gfx950", "-O3", "-fPIC", "-std=c++17",
    # keep the compiler away from packed fp32 instructions
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-munsafe-fp-atomics", "-Wall", "-Wno-unused-function",
]


def sources_sha256() -> str:
    """SHA-256 over every file of csrc/ and the public header, in name order.
    The library carries it (moe_build_sources_sha256) so that the binding can
    refuse a binary built from other sources."""
    h = hashlib.sha256()
    names = sorted(n for n in os.listdir(CSRC) if n.endswith((".hip", ".hpp", ".cpp", ".h")))
    for n in names:
        h.update(n.encode())
        with open(os.path.join(CSRC, n), "rb") as fh:
            h.update(fh.read())
    with open(HEADER, "rb") as fh:
        h.update(fh.read())
    return h.hexdigest()


# Host-only AddressSanitizer + UndefinedBehaviorSanitizer: each -fsanitize
# applies to the host compilation only (the kernels are built as usual).
SAN_HOST = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
            "-Xarch_host", "-fno-sanitize-recover=undefined",
            "-Xarch_host", "-fno-omit-frame-pointer", "-Xarch_host", "-g"]
BUILD_SAN = os.path.join(HERE, "_build_san")
OUT_SAN = os.path.join(BUILD_SAN, "libmoeffn_san.so")


def _compile(src: str, sha: str, build_dir: str = BUILD, extra=()) -> str:
    obj = os.path.join(build_dir, os.path.splitext(src)[0] + ".o")
    cmd = [HIPCC, *FLAGS, *extra, f'-DMOE_SOURCES_SHA256="{sha}"', "-x", "hip", "-c",
           os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stderr}")
    return obj


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    sha = sources_sha256()
    with ThreadPoolExecutor(max_workers=min(len(SOURCES), 8)) as ex:
        objs = list(ex.map(lambda s: _compile(s, sha), SOURCES))
    tmp = OUT + ".tmp"
    cmd = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr}")
    os.replace(tmp, OUT)
    if verbose:
        print("built", OUT)
    return OUT


def build_sanitized(verbose: bool = False) -> str:
    """The same library with the host code (argument checks, workspace
    layout, launch set-up) built under ASan + UBSan, for the CPU tests; it is
    loaded through MOEFFN_LIB with the sanitizer runtime preloaded."""
    os.makedirs(BUILD_SAN, exist_ok=True)
    sha = sources_sha256()
    with ThreadPoolExecutor(max_workers=min(len(SOURCES), 8)) as ex:
        objs = list(ex.map(lambda s: _compile(s, sha, BUILD_SAN, SAN_HOST), SOURCES))
    tmp = OUT_SAN + ".tmp"
    cmd = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-Xarch_host", "-fsanitize=address",
           "-Xarch_host", "-fsanitize=undefined", "-Xarch_host", "-shared-libsan", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr}")
    os.replace(tmp, OUT_SAN)
    if verbose:
        print("built", OUT_SAN)
    return OUT_SAN


if __name__ == "__main__":
    build(verbose=True)
