"""Build libzo.so in-tree for gfx950 with hipcc.

Every translation unit under csrc/ is compiled as HIP for gfx950 and linked
into zeroth_order_fine_amd/libzo.so, except peaks.hip (microbenchmarks used by
bench.py only), which becomes libzo_peaks.so.  Packed-fp32 VALU instructions are
disabled for all device code.
"""
import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
OUT = os.path.join(HERE, "libzo.so")
BUILD_DIR = os.path.join(HERE, "_build")
SOURCES = ["rng.hip", "gemm.hip", "layers.hip", "attention.hip", "decode.hip", "zo_api.cpp"]
# microbenchmarks for the measured ceilings bench.py reports (a library of their own)
PEAKS_SOURCE = "peaks.hip"
PEAKS_OUT = os.path.join(HERE, "libzo_peaks.so")
ARCH = "gfx950"
ROCM_LIB = "/opt/rocm/lib"
ROCTX_LINK = ["-L" + ROCM_LIB, "-lrocprofiler-sdk-roctx", "-Wl,-rpath," + ROCM_LIB]


def hipcc():
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if c and os.path.exists(c):
            return c
    raise RuntimeError("hipcc not found: the HIP library cannot be built")


def _flags():
    return ["-x", "hip", "--offload-arch=" + ARCH, "-O3", "-std=c++17", "-fPIC",
            "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
            "-I" + os.path.join(ROOT, "include"), "-I" + CSRC, "-Wno-unused-command-line-argument"]


def build(verbose=False):
    """Compile all sources (always) and link libzo.so; returns its path."""
    os.makedirs(BUILD_DIR, exist_ok=True)
    cc = hipcc()

    def compile_one(src):
        obj = os.path.join(BUILD_DIR, os.path.splitext(src)[0] + ".o")
        cmd = [cc] + _flags() + ["-c", os.path.join(CSRC, src), "-o", obj]
        r = subprocess.run(cmd, capture_output=True, text=True)
        if r.returncode != 0:
            raise RuntimeError("hipcc failed for %s:\n%s" % (src, r.stderr[-4000:]))
        if verbose and r.stderr.strip():
            sys.stderr.write(r.stderr)
        return obj

    with ThreadPoolExecutor(max_workers=min(len(SOURCES) + 1, os.cpu_count() or 4)) as ex:
        objs = list(ex.map(compile_one, SOURCES + [PEAKS_SOURCE]))
    for out, parts in ((OUT, objs[:-1]), (PEAKS_OUT, objs[-1:])):
        tmp = out + ".tmp%d" % os.getpid()
        cmd = [cc, "--offload-arch=" + ARCH, "-shared", "-fPIC", "-o", tmp] + parts
        if out == OUT:   # roctx ranges around the public calls
            cmd += ROCTX_LINK
        r = subprocess.run(cmd, capture_output=True, text=True)
        if r.returncode != 0:
            raise RuntimeError("link failed:\n" + r.stderr[-4000:])
        os.replace(tmp, out)
    return OUT


if __name__ == "__main__":
    print(build(verbose=True))
