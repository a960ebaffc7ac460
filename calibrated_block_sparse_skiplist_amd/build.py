"""Build libcalibatt.so in-tree with hipcc for gfx950.

Usage: python -m calibrated_block_sparse_skiplist_amd.build   (or build() from Python)

Every HIP source in csrc/ is compiled to an object in parallel, then linked
into calibrated_block_sparse_skiplist_amd/libcalibatt.so. The library carries
gfx950 code only.
"""
from __future__ import annotations

import concurrent.futures
import os
import shutil
import subprocess
import sys

PKG_DIR = os.path.dirname(os.path.abspath(__file__))
REPO = os.path.dirname(PKG_DIR)
CSRC = os.path.join(PKG_DIR, "csrc")
INCLUDE = os.path.join(REPO, "include")
BUILD_DIR = os.path.join(REPO, "_build")
LIB_PATH = os.path.join(PKG_DIR, "libcalibatt.so")

ARCH = "gfx950"
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = [
    "-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
    # Packed fp32 VALU forms stay disabled: the scalar fp32 forms are used throughout.
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # MFMA results in VGPRs, not AGPRs: the score accumulators are read by VALU
    # work (exponentials), and an AGPR operand costs a v_accvgpr_read first
    # (the block-energy kernel: 32 per stage and wave, and one wave less per SIMD).
    "-mllvm", "-amdgpu-mfma-vgpr-form",
    "-Wno-unused-result", "-Wno-unused-command-line-argument",
    "-I", INCLUDE, "-I", CSRC,
]


# Host-side sanitizer build (address + undefined behaviour) of the same sources,
# for CPU runs of the host logic (argument checks, list validation). Every
# sanitizer flag applies to the host compilation only (-Xarch_host): the device
# code is the ordinary gfx950 code.
SANITIZE_FLAGS = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
                  "-Xarch_host", "-fno-sanitize-recover=undefined", "-Xarch_host", "-fno-omit-frame-pointer",
                  "-Xarch_host", "-shared-libasan"]
SANITIZED_LIB = os.path.join(BUILD_DIR, "sanitized", "libcalibatt.so")


def sources() -> list[str]:
    return sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC) if f.endswith(".hip"))


def _compile(src: str, extra: list[str], out_dir: str = BUILD_DIR) -> str:
    obj = os.path.join(out_dir, os.path.basename(src).replace(".hip", ".o"))
    cmd = [HIPCC, *FLAGS, *extra, "-c", src, "-o", obj]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{' '.join(cmd)}\n{res.stdout}\n{res.stderr}")
    return obj


def build(verbose: bool = False, extra_flags: list[str] | None = None) -> str:
    """Compile every HIP source and link libcalibatt.so; returns its path."""
    if not os.path.exists(HIPCC):
        raise RuntimeError(f"hipcc not found at {HIPCC}")
    os.makedirs(BUILD_DIR, exist_ok=True)
    extra = list(extra_flags or [])
    srcs = sources()
    with concurrent.futures.ThreadPoolExecutor(max_workers=min(8, len(srcs))) as ex:
        objs = list(ex.map(lambda s: _compile(s, extra), srcs))
    tmp = LIB_PATH + ".tmp"
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"link failed:\n{' '.join(cmd)}\n{res.stdout}\n{res.stderr}")
    os.replace(tmp, LIB_PATH)
    if verbose:
        print(f"built {LIB_PATH} from {len(srcs)} sources", file=sys.stderr)
    return LIB_PATH


def build_sanitized(verbose: bool = False) -> str:
    """The host-sanitized variant of libcalibatt.so (outside the package: never loaded by default).
    Load it with the clang ASan runtime preloaded and CALIBATT_LIB set to the returned path."""
    out_dir = os.path.dirname(SANITIZED_LIB)
    os.makedirs(out_dir, exist_ok=True)
    srcs = sources()
    with concurrent.futures.ThreadPoolExecutor(max_workers=min(8, len(srcs))) as ex:
        objs = list(ex.map(lambda s: _compile(s, SANITIZE_FLAGS, out_dir), srcs))
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", *SANITIZE_FLAGS, "-o", SANITIZED_LIB, *objs]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"link failed:\n{' '.join(cmd)}\n{res.stdout}\n{res.stderr}")
    if verbose:
        print(f"built {SANITIZED_LIB}", file=sys.stderr)
    return SANITIZED_LIB


def asan_runtime() -> str:
    """Path of the clang ASan runtime that the sanitized library links against."""
    res = subprocess.run([os.path.join(os.path.dirname(os.path.realpath(HIPCC)), "..", "llvm", "bin", "clang"),
                          "-print-file-name=libclang_rt.asan-x86_64.so"], capture_output=True, text=True)
    path = res.stdout.strip()
    if res.returncode != 0 or not os.path.isabs(path) or not os.path.exists(path):
        raise RuntimeError("clang ASan runtime not found")
    return path


def clean() -> None:
    shutil.rmtree(BUILD_DIR, ignore_errors=True)


if __name__ == "__main__":
    build(verbose=True)
