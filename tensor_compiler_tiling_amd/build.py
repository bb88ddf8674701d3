"""Build libconvtile.so (HIP kernels for gfx950 + the C-ABI runtime) in-tree.

    python -m tensor_compiler_tiling_amd.build [--host-check]

Every source under csrc/ is compiled with hipcc for gfx950 into _build/ and
linked into tensor_compiler_tiling_amd/libconvtile.so.

build_host_check() also compiles every source host-only (no device code)
with AddressSanitizer and UndefinedBehaviorSanitizer and links it with
tests/sanitize/host_check.cpp into _build/asan/host_check, a CPU-only check
of the runtime's host code.
"""
from __future__ import annotations

import concurrent.futures as cf
import glob
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libconvtile.so")
ARCH = "gfx950"

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
COMMON = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
          # packed fp32 arithmetic stays off: plain fp32 code only
          "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
          "-Wall", "-Wno-unused-function", "-Wno-unused-variable",
          "-Wno-unused-command-line-argument",
          "-I", os.path.join(ROOT, "include"), "-I", CSRC]


def _compile(src: str) -> str:
    obj = os.path.join(BUILD, os.path.basename(src) + ".o")
    cmd = [HIPCC] + COMMON + ["-c", src, "-o", obj]
    if src.endswith(".cpp"):
        cmd = [HIPCC] + COMMON + ["-x", "hip", "-c", src, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stderr}")
    if r.stderr.strip():
        # keep warnings visible but terse (the host pass notes the packed-fp32 flag)
        lines = [l for l in r.stderr.splitlines() if "packed-fp32-ops" not in l and l.strip()]
        if lines:
            sys.stderr.write("\n".join(lines[:40]) + "\n")
    return obj


def build(jobs: int | None = None) -> str:
    os.makedirs(BUILD, exist_ok=True)
    srcs = sorted(glob.glob(os.path.join(CSRC, "*.hip")) + glob.glob(os.path.join(CSRC, "*.cpp")))
    jobs = jobs or min(8, os.cpu_count() or 4)
    with cf.ThreadPoolExecutor(jobs) as ex:
        objs = list(ex.map(_compile, srcs))
    tmp = LIB + ".tmp"
    # -z defs: a symbol left undefined (a kernel whose host stub was not
    # emitted, say) fails the link instead of the first load
    cmd = [HIPCC, "-shared", "-fPIC", f"--offload-arch={ARCH}", "-Wl,-z,defs", "-o", tmp] + objs
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr}")
    os.replace(tmp, LIB)
    return LIB


ASAN_DIR = os.path.join(BUILD, "asan")
HOST_CHECK = os.path.join(ASAN_DIR, "host_check")
HOST_CHECK_SRC = os.path.join(ROOT, "tests", "sanitize", "host_check.cpp")
RUNTIME_SRC = os.path.join(CSRC, "runtime.cpp")
# sanitizers on the host side only: the device code is built as usual
SANITIZE = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
            "-Xarch_host", "-fno-sanitize-recover=undefined", "-Xarch_host", "-fno-omit-frame-pointer"]


def build_host_check() -> str:
    """The host-code check binary: the C-ABI runtime (runtime.cpp, all of the
    library's host logic) built with AddressSanitizer and
    UndefinedBehaviorSanitizer on its host side, linked with the kernel
    objects of the regular build and tests/sanitize/host_check.cpp."""
    os.makedirs(ASAN_DIR, exist_ok=True)
    kernels = sorted(glob.glob(os.path.join(CSRC, "*.hip")))
    objs = [os.path.join(BUILD, os.path.basename(k) + ".o") for k in kernels]
    if not all(os.path.exists(o) for o in objs):
        build()
    flags = ["-O1", "-g", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
             "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
             "-Wno-unused-command-line-argument", "-I", os.path.join(ROOT, "include"), "-I", CSRC]
    rt_obj = os.path.join(ASAN_DIR, "runtime.cpp.o")
    main_obj = os.path.join(ASAN_DIR, "host_check.o")
    for cmd in ([HIPCC] + flags + SANITIZE + ["-x", "hip", "-c", RUNTIME_SRC, "-o", rt_obj],
                [HIPCC] + flags + SANITIZE + ["-c", HOST_CHECK_SRC, "-o", main_obj]):
        r = subprocess.run(cmd, capture_output=True, text=True)
        if r.returncode != 0:
            raise RuntimeError(f"sanitized host build failed:\n{r.stderr}")
    tmp = HOST_CHECK + ".tmp"
    r = subprocess.run([HIPCC, f"--offload-arch={ARCH}"] + SANITIZE + ["-o", tmp, main_obj, rt_obj] + objs,
                       capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"host check link failed:\n{r.stderr}")
    os.replace(tmp, HOST_CHECK)
    return HOST_CHECK


if __name__ == "__main__":
    print(build())
    if "--host-check" in sys.argv:
        print(build_host_check())
