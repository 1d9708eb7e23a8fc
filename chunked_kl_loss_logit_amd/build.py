"""Build libkdloss.so in-tree with hipcc for gfx950.

    python -m chunked_kl_loss_logit_amd.build        # or build() from Python

Every source under csrc/ is compiled (in parallel) to _build/*.o and linked
into chunked_kl_loss_logit_amd/libkdloss.so.
"""
from __future__ import annotations

import concurrent.futures as fut
import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
BUILD = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "libkdloss.so")
ARCH = "gfx950"


def _hipcc() -> str:
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if c and os.path.exists(c):
            return c
    raise RuntimeError("hipcc not found (ROCm is required to build libkdloss)")


def sources():
    return sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC) if f.endswith((".hip", ".cpp")))


def _flags():
    return [
        f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
        "-I", os.path.join(ROOT, "include"), "-I", CSRC,
        # keep hipcc from forming packed fp32 VALU ops on its own
        "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
        "-Wno-unused-command-line-argument",
    ]


def _compile(src: str, verbose: bool) -> str:
    obj = os.path.join(BUILD, os.path.basename(src) + ".o")
    cmd = [_hipcc(), *_flags(), "-c", src, "-o", obj]
    if src.endswith(".cpp"):
        cmd.insert(1, "-xhip")
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {os.path.basename(src)}:\n{r.stdout}\n{r.stderr}")
    if verbose:
        noise = "not a recognized feature for this target"
        msg = "\n".join(l for l in (r.stdout + r.stderr).splitlines() if noise not in l)
        if msg.strip():
            print(msg)
    return obj


def build(verbose: bool = False) -> str:
    """Compile every source and link libkdloss.so; returns the library path."""
    os.makedirs(BUILD, exist_ok=True)
    srcs = sources()
    jobs = max(1, min(len(srcs), int(os.environ.get("MAX_JOBS", os.cpu_count() or 1)), 16))
    with fut.ThreadPoolExecutor(jobs) as ex:
        objs = list(ex.map(lambda s: _compile(s, verbose), srcs))
    tmp = LIB + ".tmp"
    cmd = [_hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, LIB)
    return LIB


# ---------------------------------------------------------------- host sanitizer build
# The host code of the C ABI (argument checks, workspace planning, launch
# sequences) compiled with the address and undefined-behaviour sanitizers,
# linked with the uninstrumented kernels and a driver that runs the ABI's
# rejection and workspace-size cases on the CPU (tests/host/abi_driver.cpp).
ASAN_DIR = os.path.join(BUILD, "host_sanitizers")
ASAN_HOST = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
             "-Xarch_host", "-fno-sanitize-recover=undefined", "-Xarch_host", "-fno-omit-frame-pointer"]


def build_host_sanitizer_driver() -> str:
    """Build the sanitizer-instrumented ABI driver; returns its path.  Needs
    the kernels' objects of a regular build (build() makes them)."""
    os.makedirs(ASAN_DIR, exist_ok=True)
    api = os.path.join(CSRC, "kd_api.cpp")
    kernels = [os.path.join(BUILD, os.path.basename(s) + ".o") for s in sources() if s.endswith(".hip")]
    missing = [k for k in kernels if not os.path.exists(k)]
    if missing:
        build()
    api_o = os.path.join(ASAN_DIR, "kd_api.o")
    drv_src = os.path.join(ROOT, "tests", "host", "abi_driver.cpp")
    drv_o = os.path.join(ASAN_DIR, "abi_driver.o")
    exe = os.path.join(ASAN_DIR, "abi_driver")
    flags = [f for f in _flags() if f != "-O3"] + ["-O1", "-g"]
    steps = [
        [_hipcc(), "-xhip", *flags, *ASAN_HOST, "-c", api, "-o", api_o],
        [_hipcc(), *flags, *ASAN_HOST, "-c", drv_src, "-o", drv_o],
        [_hipcc(), f"--offload-arch={ARCH}", *ASAN_HOST, "-o", exe, drv_o, api_o, *kernels],
    ]
    for cmd in steps:
        r = subprocess.run(cmd, capture_output=True, text=True)
        if r.returncode != 0:
            raise RuntimeError(f"sanitizer build failed:\n{' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    return exe


if __name__ == "__main__":
    path = build(verbose="-v" in sys.argv)
    print(path)
