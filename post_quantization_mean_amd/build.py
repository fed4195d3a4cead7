"""Builds libawq_mi355x.so (the C ABI of include/awq.h) in-tree with hipcc for gfx950.

    python -m post_quantization_mean_amd.build [-v] [--sanitize]
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
BUILD_DIR = os.path.join(ROOT, "_build")
LIB_NAME = "libawq_mi355x.so"
LIB_PATH = os.path.join(PKG, LIB_NAME)
ARCH = "gfx950"

SOURCES = ["act_stats.hip", "scales.hip", "quant.hip", "err_gemm.hip", "export.hip", "variants.hip", "w4a16.hip", "block_gemm.hip", "gram.hip", "abi.hip"]

COMMON_FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-fvisibility=hidden",
    "-Wall", "-Wno-unused-function",
    # no packed fp32 instructions in device code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    f"-I{INCLUDE}", f"-I{CSRC}",
]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found: the HIP library cannot be built")


def _run(cmd: list[str], verbose: bool) -> None:
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    out = (r.stdout + r.stderr).strip()
    # the host pass does not know the device-only feature above; that warning is harmless
    lines = [l for l in out.splitlines() if "packed-fp32-ops" not in l]
    if r.returncode != 0:
        raise RuntimeError(f"command failed ({r.returncode}): {' '.join(cmd)}\n" + "\n".join(lines))
    if verbose and lines:
        print("\n".join(lines), flush=True)


# host code only: the device code of a sanitized build is the same as the product's
SANITIZE_FLAGS = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
                  "-Xarch_host", "-fno-omit-frame-pointer", "-Xarch_host", "-fno-sanitize-recover=undefined"]
SANITIZED_LIB_PATH = os.path.join(BUILD_DIR, "sanitized", "libawq_mi355x_asan_ubsan.so")


def build(verbose: bool = False, jobs: int | None = None, sanitize: bool = False) -> str:
    """Compiles every HIP source for gfx950 and links the shared library. Always rebuilds.

    With `sanitize`, the host code is built with AddressSanitizer and UndefinedBehaviorSanitizer
    into a separate library under the build folder (for host-side checks of the C ABI; load it
    with the sanitizer runtime preloaded)."""
    cc = hipcc()
    out_dir = os.path.dirname(SANITIZED_LIB_PATH) if sanitize else BUILD_DIR
    lib_path = SANITIZED_LIB_PATH if sanitize else LIB_PATH
    extra = SANITIZE_FLAGS if sanitize else []
    os.makedirs(out_dir, exist_ok=True)
    objs = []

    def compile_one(src: str) -> str:
        obj = os.path.join(out_dir, src.replace(".hip", ".o"))
        _run([cc, *COMMON_FLAGS, *extra, "-c", os.path.join(CSRC, src), "-o", obj], verbose)
        return obj

    with cf.ThreadPoolExecutor(jobs or min(len(SOURCES), os.cpu_count() or 1)) as ex:
        objs = list(ex.map(compile_one, SOURCES))
    tmp = lib_path + ".tmp"
    _run([cc, f"--offload-arch={ARCH}", "-shared", "-fPIC", *extra, "-o", tmp, *objs], verbose)
    os.replace(tmp, lib_path)
    return lib_path


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv, sanitize="--sanitize" in sys.argv))
