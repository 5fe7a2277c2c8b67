"""Builds libavae.so in-tree for gfx950 with hipcc (one object per source,
compiled in parallel, then linked).  Run as ``python -m
bigvgan_waveform_decoder_amd.build``."""
from __future__ import annotations

import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
OUT = os.path.join(PKG, "libavae.so")
BUILD_DIR = os.path.join(ROOT, "_build")
ARCH = os.environ.get("AVAE_OFFLOAD_ARCH", "gfx950")

COMMON = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-Wall",
    # no packed-FP32 instructions in device code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", os.path.join(ROOT, "include"),
]


def hipcc() -> str:
    exe = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(exe):
        raise RuntimeError("hipcc not found (ROCm is required to build libavae.so)")
    return exe


def sources():
    return sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC)
                  if f.endswith((".hip", ".cpp")))


def _compile(src: str) -> str:
    obj = os.path.join(BUILD_DIR, os.path.basename(src) + ".o")
    cmd = [hipcc(), *COMMON, "-c", src, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"compile failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    return obj


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD_DIR, exist_ok=True)
    srcs = sources()
    with cf.ThreadPoolExecutor(max_workers=min(8, len(srcs))) as ex:
        objs = list(ex.map(_compile, srcs))
    tmp = OUT + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, OUT)
    if verbose:
        print(f"built {OUT}")
    return OUT


# Host-sanitized variant (a check of the C-ABI's host code, not a product):
# the host parts of the C++ sources (argument checks, planning, the launch
# profiler) built with the address and undefined-behaviour sanitizers, linked
# with the regular kernel objects.  Device code is never sanitized.
HOST_SAN = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
            "-Xarch_host", "-fno-sanitize-recover=all", "-Xarch_host", "-fno-omit-frame-pointer"]
SAN_OUT = os.path.join(BUILD_DIR, "libavae_hostsan.so")


def asan_runtime() -> str:
    """The compiler's shared ASan runtime (preloaded by the process that loads
    the host-sanitized library)."""
    clang_dir = os.path.join(os.path.dirname(os.path.realpath(hipcc())), "..", "lib", "llvm",
                             "lib", "clang")
    for root, _, files in os.walk(os.path.realpath(clang_dir)):
        if "libclang_rt.asan-x86_64.so" in files:
            return os.path.join(root, "libclang_rt.asan-x86_64.so")
    raise RuntimeError("libclang_rt.asan-x86_64.so not found next to hipcc")


def build_host_sanitized(verbose: bool = False) -> str:
    os.makedirs(BUILD_DIR, exist_ok=True)
    objs = []
    jobs = []
    for src in sources():
        if src.endswith(".cpp"):
            obj = os.path.join(BUILD_DIR, os.path.basename(src) + ".san.o")
            flags = [f"--offload-arch={ARCH}", "-O1", "-g", "-std=c++17", "-fPIC", "-Wall",
                     "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
                     "-I", os.path.join(ROOT, "include"), *HOST_SAN]
            jobs.append([hipcc(), *flags, "-c", src, "-o", obj])
            objs.append(obj)
        else:
            obj = os.path.join(BUILD_DIR, os.path.basename(src) + ".o")
            if not os.path.exists(obj) or os.path.getmtime(obj) < os.path.getmtime(src):
                jobs.append([hipcc(), *COMMON, "-c", src, "-o", obj])
            objs.append(obj)

    def run(cmd):
        r = subprocess.run(cmd, capture_output=True, text=True)
        if r.returncode != 0:
            raise RuntimeError(f"compile failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    with cf.ThreadPoolExecutor(max_workers=min(8, max(len(jobs), 1))) as ex:
        list(ex.map(run, jobs))
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-shared-libasan", *HOST_SAN,
           "-o", SAN_OUT, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    if verbose:
        print(f"built {SAN_OUT}")
    return SAN_OUT


if __name__ == "__main__":
    if "--host-sanitized" in sys.argv[1:]:
        build_host_sanitized(verbose=True)
    else:
        build(verbose=True)
    sys.exit(0)
