"""Build libfno.so in-tree with hipcc for gfx950.

Usage: python -m fno_spectral_convolution_amd.build   (or call build()).
Each HIP source compiles to an object of its own (in parallel, up to FNO_BUILD_JOBS or the
CPU count, at most 8), then one hipcc line links the shared library.
"""
from __future__ import annotations

import concurrent.futures
import glob
import os
import shutil
import subprocess
import sys
import tempfile

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libfno.so")

HIPCC_FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
    # packed fp32 VALU instructions stay off in every HIP translation unit
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function",
]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found")


def sources():
    return sorted(glob.glob(os.path.join(CSRC, "*.hip")))


def _run(cmd):
    res = subprocess.run(cmd, capture_output=True, text=True)
    out = "\n".join(line for line in (res.stdout + res.stderr).splitlines()
                    if "packed-fp32-ops" not in line)
    return res.returncode, out


def _jobs() -> int:
    env = os.environ.get("FNO_BUILD_JOBS")
    if env:
        return max(1, int(env))
    return max(1, min(8, os.cpu_count() or 1))


def build(verbose: bool = False) -> str:
    """Compile every HIP source of libfno into one shared library (always recompiles)."""
    cc = hipcc()
    tmp = LIB + ".tmp"
    with tempfile.TemporaryDirectory(prefix="libfno_build_") as obj_dir:
        cmds = []
        for src in sources():
            obj = os.path.join(obj_dir, os.path.basename(src) + ".o")
            cmds.append([cc] + HIPCC_FLAGS + ["-I", INCLUDE, "-I", CSRC, "-c", src, "-o", obj])
        with concurrent.futures.ThreadPoolExecutor(max_workers=_jobs()) as pool:
            results = list(pool.map(_run, cmds))
        for cmd, (rc, out) in zip(cmds, results):
            if verbose:
                print(" ".join(cmd), flush=True)
            if rc != 0:
                raise RuntimeError(f"hipcc failed ({rc}) on {cmd[-3]}:\n{out}")
            if verbose and out.strip():
                print(out)
        link = [cc, "--offload-arch=gfx950", "-fPIC", "-shared"] + [c[-1] for c in cmds] + \
            ["-o", tmp]
        if verbose:
            print(" ".join(link), flush=True)
        rc, out = _run(link)
        if rc != 0:
            raise RuntimeError(f"hipcc link failed ({rc}):\n{out}")
    os.replace(tmp, LIB)
    return LIB


SAN_LIB = os.path.join(ROOT, "_build", "libfno_sanitize.so")

# host-side AddressSanitizer + UndefinedBehaviorSanitizer: each -fsanitize goes to the host
# compilation only (-Xarch_host); the device code is built as in the product library
SAN_FLAGS = [
    "--offload-arch=gfx950", "-O1", "-g", "-std=c++17", "-fPIC",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
    "-Xarch_host", "-fno-omit-frame-pointer", "-Xarch_host", "-fno-sanitize-recover=all",
    "-Wno-unused-function",
]


def build_sanitized(verbose: bool = False) -> str:
    """libfno's host code (descriptor validation, float64 table build, workspace layout, the
    Tucker planner, every entry point's argument checks) built with host ASan + UBSan into
    _build/libfno_sanitize.so, for CPU-only checks of the host logic; it is loaded into a
    Python process with the sanitizer runtime preloaded (see sanitizer_runtime())."""
    cc = hipcc()
    os.makedirs(os.path.dirname(SAN_LIB), exist_ok=True)
    with tempfile.TemporaryDirectory(prefix="libfno_san_") as obj_dir:
        cmds = []
        for src in sources():
            obj = os.path.join(obj_dir, os.path.basename(src) + ".o")
            cmds.append([cc] + SAN_FLAGS + ["-I", INCLUDE, "-I", CSRC, "-c", src, "-o", obj])
        with concurrent.futures.ThreadPoolExecutor(max_workers=_jobs()) as pool:
            results = list(pool.map(_run, cmds))
        for cmd, (rc, out) in zip(cmds, results):
            if verbose:
                print(" ".join(cmd), flush=True)
            if rc != 0:
                raise RuntimeError(f"hipcc (sanitized) failed ({rc}) on {cmd[-3]}:\n{out}")
        link = [cc, "--offload-arch=gfx950", "-fPIC", "-shared", "-Xarch_host",
                "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined"] + \
            [c[-1] for c in cmds] + ["-o", SAN_LIB + ".tmp"]
        rc, out = _run(link)
        if rc != 0:
            raise RuntimeError(f"hipcc (sanitized) link failed ({rc}):\n{out}")
    os.replace(SAN_LIB + ".tmp", SAN_LIB)
    return SAN_LIB


def sanitizer_runtime() -> str:
    """Path of the compiler's AddressSanitizer runtime (to preload into an uninstrumented
    Python process that loads the sanitized library)."""
    res = subprocess.run([hipcc(), "-print-file-name=libclang_rt.asan-x86_64.so"],
                         capture_output=True, text=True)
    path = res.stdout.strip()
    if res.returncode != 0 or not os.path.isabs(path) or not os.path.exists(path):
        # the runtime sits next to the compiler's resource directory
        res = subprocess.run([hipcc(), "-print-resource-dir"], capture_output=True, text=True)
        path = os.path.join(res.stdout.strip(), "lib", "linux", "libclang_rt.asan-x86_64.so")
    if not os.path.exists(path):
        raise RuntimeError("AddressSanitizer runtime not found")
    return path


if __name__ == "__main__":
    if "--sanitize" in sys.argv:
        print(build_sanitized(verbose="-v" in sys.argv))
    else:
        print(build(verbose="-v" in sys.argv))
