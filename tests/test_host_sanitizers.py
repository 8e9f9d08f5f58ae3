"""The host runtime (zo_api.cpp) under AddressSanitizer and UndefinedBehaviorSanitizer.

The packing tables, the workspace bump allocator, the side-operand geometry and the
bank's key and offset arithmetic all run on the host; tests/sanitize/zo_host_driver.cpp
drives them through the C-ABI on seeded random batches, plans and banks (and the error
paths of the device calls, which return before any launch).  The runtime and the driver
are compiled with the sanitizers on their host code only (device code is the library's
usual build) and linked into one executable, which must exit 0 with no report.
No GPU is needed."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PKG = os.path.join(ROOT, "zeroth_order_fine_amd")
BUILD = os.path.join(PKG, "_build")
OUT = os.path.join(BUILD, "sanitize")


def _hipcc():
    for c in ("/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if c and os.path.exists(c):
            return c
    pytest.skip("hipcc not available")


def test_host_runtime_clean_under_asan_and_ubsan():
    from zeroth_order_fine_amd import build as zbuild
    objs = [os.path.join(BUILD, n) for n in ("rng.o", "gemm.o", "layers.o", "attention.o", "decode.o")]
    if not all(os.path.exists(o) for o in objs):
        zbuild.build()
    os.makedirs(OUT, exist_ok=True)
    cc = _hipcc()
    # sanitizer flags apply to the host compilation only
    san = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
           "-Xarch_host", "-fno-sanitize-recover=undefined", "-Xarch_host", "-fno-omit-frame-pointer"]
    flags = ["-x", "hip", "--offload-arch=gfx950", "-O1", "-g", "-std=c++17", "-fPIC",
             "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
             "-I" + os.path.join(ROOT, "include"), "-I" + os.path.join(PKG, "csrc"),
             "-Wno-unused-command-line-argument"]
    api_o = os.path.join(OUT, "zo_api_san.o")
    drv_o = os.path.join(OUT, "driver_san.o")
    exe = os.path.join(OUT, "zo_host_driver")
    for src, obj in ((os.path.join(PKG, "csrc", "zo_api.cpp"), api_o),
                     (os.path.join(ROOT, "tests", "sanitize", "zo_host_driver.cpp"), drv_o)):
        r = subprocess.run([cc] + flags + san + ["-c", src, "-o", obj], capture_output=True, text=True)
        assert r.returncode == 0, r.stderr[-3000:]
    r = subprocess.run([cc, "--offload-arch=gfx950"] + san + [drv_o, api_o] + objs + zbuild.ROCTX_LINK + ["-o", exe],
                       capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-3000:]
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=0:exitcode=23",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1", HIP_VISIBLE_DEVICES="")
    r = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=600)
    out = r.stdout + r.stderr
    assert r.returncode == 0, out[-4000:]
    assert "ERROR: AddressSanitizer" not in out and "runtime error" not in out, out[-4000:]
    assert "0 failed expectations" in out, out[-2000:]
