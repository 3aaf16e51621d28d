"""Build libmxfp4.so in-tree with hipcc for gfx950 (no GPU needed to compile).

    python -m mxfp4_block_scaled_02_amd.build
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libmxfp4.so")
SOURCES = ["quant.hip", "rmsnorm_quant.hip", "pack_b.hip", "gemm.hip", "nvfp4.hip"]

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
    # no packed-fp32 VALU instructions in device code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function",
    "-I", os.path.join(ROOT, "include"),
]


# Host-side AddressSanitizer + UndefinedBehaviorSanitizer instrumentation for a
# CPU-only check build (the validation paths of every entry point run before
# any HIP call). Each -fsanitize applies to the host pass only; device code is
# built exactly as in the normal library.
SAN_FLAGS = [
    "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
    "-Xarch_host", "-fno-sanitize-recover=undefined", "-Xarch_host", "-fno-omit-frame-pointer", "-g",
]
SAN_BUILD = os.path.join(BUILD, "sanitized")
SAN_LIB = os.path.join(SAN_BUILD, "libmxfp4_sanitized.so")


def _compile(src: str, outdir: str = BUILD, extra=()) -> str:
    obj = os.path.join(outdir, os.path.splitext(src)[0] + ".o")
    cmd = [HIPCC, *FLAGS, *extra, "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stdout}\n{r.stderr}")
    return obj


def _link(objs, out, extra=()):
    tmp = out + ".tmp"
    cmd = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", *extra, *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, out)
    return out


def build(verbose: bool = True) -> str:
    """Compile every HIP source and link libmxfp4.so; always rebuilds."""
    os.makedirs(BUILD, exist_ok=True)
    with cf.ThreadPoolExecutor(max_workers=min(4, len(SOURCES))) as ex:
        objs = list(ex.map(_compile, SOURCES))
    _link(objs, LIB)
    if verbose:
        print(f"built {LIB}")
    return LIB


def build_sanitized(verbose: bool = True) -> str:
    """The same library with ASan + UBSan on its host code (for CPU-side checks only;
    load it with the clang ASan runtime preloaded, see sanitizer_runtime())."""
    os.makedirs(SAN_BUILD, exist_ok=True)
    with cf.ThreadPoolExecutor(max_workers=min(4, len(SOURCES))) as ex:
        objs = list(ex.map(lambda s: _compile(s, SAN_BUILD, SAN_FLAGS), SOURCES))
    _link(objs, SAN_LIB, ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
                          "-shared-libsan"])
    if verbose:
        print(f"built {SAN_LIB}")
    return SAN_LIB


def sanitizer_runtime() -> str:
    """Path of the clang ASan runtime matching hipcc (to LD_PRELOAD into an uninstrumented python)."""
    r = subprocess.run([os.path.join(os.path.dirname(os.path.realpath(HIPCC)), "..", "llvm", "bin", "clang"),
                        "-print-file-name=libclang_rt.asan-x86_64.so"], capture_output=True, text=True)
    path = r.stdout.strip()
    if r.returncode != 0 or not os.path.isabs(path) or not os.path.exists(path):
        raise RuntimeError("clang ASan runtime not found")
    return path


if __name__ == "__main__":
    if sys.argv[1:] == ["sanitized"]:
        build_sanitized()
    else:
        build()
    sys.exit(0)
