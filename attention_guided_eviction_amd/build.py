"""Compile libbkv.so (HIP, gfx950) in-tree next to this file.

    python -m attention_guided_eviction_amd.build [-q]
    python -m attention_guided_eviction_amd.build --host-sanitized [-q]

Every HIP source under csrc/ is compiled to an object (in parallel, under _build/) and
linked into one shared library exporting the C ABI of include/bkv.h.  Packed-FP32
instruction selection is disabled for device code.

--host-sanitized builds _build/libbkv_host_sanitized.so instead: the host side of the
library (argument checks, workspace sizing, overlap sweep; csrc/bkv_api.hip) with
AddressSanitizer and UndefinedBehaviorSanitizer on the host code only, linked against
launcher stubs that refuse every launch.  It serves host-only tests of the validation
code (run with the sanitizer runtime preloaded); it can launch nothing.
"""
from __future__ import annotations

import concurrent.futures as cf
import glob
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
LIB = os.path.join(PKG, "libbkv.so")
BUILD_DIR = os.path.join(PKG, "_build")
HOST_SANITIZED_LIB = os.path.join(BUILD_DIR, "libbkv_host_sanitized.so")
ARCH = "gfx950"


def rocm() -> str:
    return os.environ.get("ROCM_PATH", "/opt/rocm")


def hipcc() -> str:
    p = os.path.join(rocm(), "bin", "hipcc")
    return p if os.path.exists(p) else "hipcc"


def sources():
    return sorted(glob.glob(os.path.join(PKG, "csrc", "*.hip")))


COMMON = ["-O3", "-std=c++17", "-fPIC", "-Wall", "-Wno-unused-result"]
DEVICE = [f"--offload-arch={ARCH}", "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]


def _includes():
    return ["-I", os.path.join(ROOT, "include"), "-I", os.path.join(PKG, "csrc")]


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    out = (r.stdout + r.stderr).strip()
    if r.returncode != 0:
        raise RuntimeError("hipcc failed:\n" + " ".join(cmd) + "\n" + out)
    # The host pass does not know the device-only target feature; that warning is expected.
    noise = [ln for ln in out.splitlines() if "packed-fp32-ops" not in ln and ln.strip()]
    if verbose and noise:
        print("\n".join(noise), flush=True)


def _compile_all(jobs, verbose):
    workers = max(1, min(len(jobs), int(os.environ.get("MAX_JOBS", os.cpu_count() or 1)), 16))
    with cf.ThreadPoolExecutor(workers) as ex:
        for f in [ex.submit(_run, cmd, verbose) for cmd in jobs]:
            f.result()


def build(verbose: bool = False) -> str:
    """Compile every source into libbkv.so (always recompiles).  Returns the path."""
    os.makedirs(BUILD_DIR, exist_ok=True)
    objs, jobs = [], []
    for src in sources():
        obj = os.path.join(BUILD_DIR, os.path.basename(src)[:-4] + ".o")
        objs.append(obj)
        jobs.append([hipcc(), "-c", "-x", "hip"] + DEVICE + COMMON + _includes() + ["-o", obj, src])
    _compile_all(jobs, verbose)
    tmp = LIB + ".tmp"
    _run([hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp] + objs, verbose)
    os.replace(tmp, LIB)
    return LIB


def sanitizer_runtime() -> str:
    """The compiler's AddressSanitizer runtime (to preload into a host process that loads
    the sanitized library)."""
    hits = sorted(glob.glob(os.path.join(rocm(), "llvm", "lib", "clang", "*", "lib", "linux",
                                         "libclang_rt.asan-x86_64.so")))
    if not hits:
        raise RuntimeError("no libclang_rt.asan-x86_64.so under " + rocm())
    return hits[-1]


STUBS = os.path.join(PKG, "csrc", "host_only", "launch_stubs.cpp")


def build_host_sanitized(verbose: bool = False) -> str:
    """The host-only, sanitizer-instrumented library (see the module docstring)."""
    os.makedirs(BUILD_DIR, exist_ok=True)
    san = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
           "-Xarch_host", "-fno-sanitize-recover=undefined", "-Xarch_host", "-fno-omit-frame-pointer",
           "-Xarch_host", "-shared-libsan"]
    objs, jobs = [], []
    for src in (os.path.join(PKG, "csrc", "bkv_api.hip"), STUBS):
        obj = os.path.join(BUILD_DIR, "san_" + os.path.basename(src).split(".")[0] + ".o")
        objs.append(obj)
        jobs.append([hipcc(), "-c", "-x", "hip"] + DEVICE + ["-O1", "-g"] + COMMON[1:] + san + _includes() +
                    ["-o", obj, src])
    _compile_all(jobs, verbose)
    tmp = HOST_SANITIZED_LIB + ".tmp"
    _run([hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC"] + san + ["-o", tmp] + objs, verbose)
    os.replace(tmp, HOST_SANITIZED_LIB)
    return HOST_SANITIZED_LIB


if __name__ == "__main__":
    quiet = "-q" in sys.argv
    if "--host-sanitized" in sys.argv:
        print(build_host_sanitized(verbose=not quiet))
    else:
        print(build(verbose=not quiet))
