"""libfno's host code under AddressSanitizer and UndefinedBehaviorSanitizer (CPU only).

The host side of the library (descriptor validation, the float64 table build and workspace
layout that fno_plan_create runs before its first HIP call, the Tucker contraction planner,
argument checks) is built with host ASan + UBSan into _build/libfno_sanitize.so and the CPU
boundary and planner tests run against it in a child Python process with the sanitizer runtime
preloaded.  Any sanitizer report fails the run (halt on error).  The sanitized build is cached
under _build/ and redone when a source or the build script changes.
"""
import hashlib
import glob
import os
import subprocess
import sys

import pytest

from fno_spectral_convolution_amd import build as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
TESTS = ["tests/test_boundary_cpu.py", "tests/test_tucker_order_cpu.py"]


def _sources_digest():
    h = hashlib.sha256()
    files = sorted(glob.glob(os.path.join(B.CSRC, "*")) + [os.path.join(B.INCLUDE, "fno.h"),
                                                         os.path.abspath(B.__file__)])
    for f in files:
        h.update(os.path.basename(f).encode())
        h.update(open(f, "rb").read())
    return h.hexdigest()


def _sanitized_library():
    stamp = B.SAN_LIB + ".sha256"
    digest = _sources_digest()
    if not (os.path.exists(B.SAN_LIB) and os.path.exists(stamp)
            and open(stamp).read().strip() == digest):
        B.build_sanitized()
        with open(stamp, "w") as f:
            f.write(digest + "\n")
    return B.SAN_LIB


def test_host_code_clean_under_sanitizers():
    import torch
    if torch.cuda.device_count() > 0:
        pytest.skip("CPU-only check: on a GPU host plan creation goes on to the device")
    lib = _sanitized_library()
    env = dict(os.environ)
    env.update({
        "LD_PRELOAD": B.sanitizer_runtime(),
        "ASAN_OPTIONS": "detect_leaks=0:halt_on_error=1:abort_on_error=0",
        "UBSAN_OPTIONS": "halt_on_error=1:print_stacktrace=1",
        "FNO_LIBRARY": lib,
    })
    res = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider"]
                         + TESTS, cwd=ROOT, env=env, capture_output=True, text=True,
                         timeout=900)
    out = res.stdout + res.stderr
    print(out[-3000:])
    assert res.returncode == 0, out[-3000:]
    assert "Sanitizer" not in out and "runtime error" not in out, out[-3000:]
    assert " passed" in out
