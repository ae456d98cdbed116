"""Host-sanitized build of libmoe.so for the CPU tests of the C ABI.

    python -m sparse_mixture_experts_02_amd.build_sanitized

Every source is compiled with AddressSanitizer and UndefinedBehaviorSanitizer on its host code
only (the device code is built as in the release library, see build.py) into _build/san/, and
linked into _build/san/libmoe_host_sanitized.so, which tests/test_host_sanitized.py loads with the
sanitizer runtime preloaded. Each sanitizer flag applies to the host pass alone (-Xarch_host
right before it). CPU only: nothing here runs on a GPU.
"""
from __future__ import annotations

import concurrent.futures
import glob
import os
import subprocess
import sys

from .build import ARCH, BUILD_DIR, COMMON_FLAGS, HIPCC, sources

SAN_DIR = os.path.join(BUILD_DIR, "san")
SAN_LIB_PATH = os.path.join(SAN_DIR, "libmoe_host_sanitized.so")
SAN_HOST_FLAGS = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
                  "-Xarch_host", "-fno-sanitize-recover=all", "-Xarch_host", "-fno-omit-frame-pointer"]


def sanitizer_runtime() -> str:
    """Path of the clang AddressSanitizer runtime the sanitized library links against ('' if absent)."""
    llvm = os.path.join(os.path.dirname(os.path.dirname(os.path.realpath(HIPCC))), "lib", "llvm")
    hits = sorted(glob.glob(os.path.join(llvm, "lib", "clang", "*", "lib", "linux", "libclang_rt.asan-x86_64.so")))
    if not hits:
        hits = sorted(glob.glob("/opt/rocm/lib/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
    return hits[-1] if hits else ""


def _compile_san(src: str) -> str:
    obj = os.path.join(SAN_DIR, os.path.basename(src) + ".o")
    flags = [f if f != "-O3" else "-O1" for f in COMMON_FLAGS]
    cmd = [HIPCC, *flags, "-g", *SAN_HOST_FLAGS, "-c", src, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stdout}\n{r.stderr}")
    return obj


def build_host_sanitized(verbose: bool = False) -> str:
    """Build the host-sanitized library (for the CPU tests of the C ABI); returns its path."""
    os.makedirs(SAN_DIR, exist_ok=True)
    srcs = sources()
    jobs = min(len(srcs), max(1, min(16, os.cpu_count() or 1)))
    with concurrent.futures.ThreadPoolExecutor(max_workers=jobs) as ex:
        objs = list(ex.map(_compile_san, srcs))
    tmp = SAN_LIB_PATH + ".tmp"
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-Xarch_host", "-fsanitize=address",
           "-Xarch_host", "-fsanitize=undefined", "-shared-libsan", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, SAN_LIB_PATH)
    if verbose:
        print(f"built {SAN_LIB_PATH} from {len(srcs)} sources (host code with ASan + UBSan)")
    return SAN_LIB_PATH


if __name__ == "__main__":
    build_host_sanitized(verbose=True)
    sys.exit(0)
