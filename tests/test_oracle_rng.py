"""Pins of the oracle's random streams (oracle/philox_normal.c).

* Philox4x32-10 block function against two independent installed
  implementations (PyTorch's header-only engine and rocRAND's device/host
  engine), each compiled and run here.
* ln, sin and cos of the exact-operation spec against mpmath at 4 ulp.
* Box-Muller output against the textbook formula evaluated in mpmath.
* the Gaussian stream's moments, a KS test and pair independence.
* the central-limit statement of the arXiv abstract of "Inference-Native
  Zeroth-Order Optimization" (factorized perturbations approach dense
  Gaussian ones as rank grows): entries of G V^T / sqrt(r) have kurtosis
  exactly 3 + 6/r.
"""
import os
import shutil
import subprocess
import tempfile

import mpmath as mp
import numpy as np
import pytest
from scipy import stats

from oracle import rng

TORCH_INC = None
try:
    import torch
    TORCH_INC = os.path.join(os.path.dirname(torch.__file__), "include")
except Exception:  # pragma: no cover
    pass


@pytest.fixture(scope="module")
def torch_philox_exe():
    if TORCH_INC is None or shutil.which("g++") is None:
        pytest.skip("torch headers or g++ missing")
    d = tempfile.mkdtemp()
    src = os.path.join(d, "p.cpp")
    with open(src, "w") as f:
        f.write("""
#include <ATen/core/PhiloxRNGEngine.h>
#include <cstdio>
#include <cstdint>
// stdin: lines "c0 c1 c2 c3 k0 k1" (hex); stdout: the block, one line each.
int main(){ unsigned c[4],k[2];
  while (scanf("%x %x %x %x %x %x",&c[0],&c[1],&c[2],&c[3],&k[0],&k[1])==6){
    uint64_t seed = (uint64_t)k[0] | ((uint64_t)k[1]<<32);
    uint64_t sub = (uint64_t)c[2] | ((uint64_t)c[3]<<32);
    uint64_t off = (uint64_t)c[0] | ((uint64_t)c[1]<<32);
    at::philox_engine e(seed, sub, off);
    unsigned a=e(),b=e(),x=e(),y=e(); printf("%08x %08x %08x %08x\\n",a,b,x,y);} }
""")
    exe = os.path.join(d, "p")
    subprocess.check_call(["g++", "-O1", "-std=c++17", "-I" + TORCH_INC, src, "-o", exe])
    return exe


def test_philox_matches_installed_engine(torch_philox_exe):
    rs = np.random.default_rng(1)
    n = 20000
    ctr = rs.integers(0, 2**32, size=(n, 4), dtype=np.uint64).astype(np.uint32)
    key = rs.integers(0, 2**32, size=(n, 2), dtype=np.uint64).astype(np.uint32)
    ctr[:4] = [[0, 0, 0, 0], [0xFFFFFFFF] * 4, [1, 2, 3, 4], [0xFFFFFFFF, 0, 0xFFFFFFFF, 0]]
    key[:4] = [[0, 0], [0xFFFFFFFF] * 2, [5, 6], [0, 0xFFFFFFFF]]
    inp = "\n".join(" ".join("%x" % v for v in list(c) + list(k)) for c, k in zip(ctr, key))
    out = subprocess.run([torch_philox_exe], input=inp, capture_output=True, text=True, check=True).stdout
    ref = np.array([[int(x, 16) for x in line.split()] for line in out.strip().splitlines()], np.uint32)
    got = rng.philox_blocks(ctr, key)
    assert np.array_equal(got, ref)


ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")


@pytest.fixture(scope="module")
def rocrand_philox_exe():
    hipcc = shutil.which("hipcc") or os.path.join(ROCM, "bin", "hipcc")
    hdr = os.path.join(ROCM, "include", "rocrand", "rocrand_philox4x32_10.h")
    if not (os.path.exists(hipcc) and os.path.exists(hdr)):
        pytest.skip("hipcc or the rocRAND headers missing")
    d = tempfile.mkdtemp()
    src = os.path.join(d, "r.cpp")
    with open(src, "w") as f:
        f.write("""
#include <rocrand/rocrand_philox4x32_10.h>
#include <cstdio>
// the engine's ten-round block function (a protected member), reached through a subclass
struct Probe : rocrand_device::philox4x32_10_engine {
  uint4 block(uint4 c, uint2 k) { return this->ten_rounds(c, k); }
};
// stdin: lines "c0 c1 c2 c3 k0 k1" (hex); stdout: the block, one line each.
int main() { unsigned c[4], k[2]; Probe p;
  while (scanf("%x %x %x %x %x %x", &c[0], &c[1], &c[2], &c[3], &k[0], &k[1]) == 6) {
    uint4 r = p.block(make_uint4(c[0], c[1], c[2], c[3]), make_uint2(k[0], k[1]));
    printf("%08x %08x %08x %08x\\n", r.x, r.y, r.z, r.w); } }
""")
    exe = os.path.join(d, "r")
    subprocess.check_call([hipcc, "-O1", "-std=c++17", "-x", "hip", "--cuda-host-only", src, "-o", exe],
                          stderr=subprocess.DEVNULL)
    return exe


def test_philox_matches_rocrand(rocrand_philox_exe):
    """The same comparison against rocRAND's engine (counter = 4 words, key = 2 words)."""
    rs = np.random.default_rng(2)
    n = 20000
    ctr = rs.integers(0, 2**32, size=(n, 4), dtype=np.uint64).astype(np.uint32)
    key = rs.integers(0, 2**32, size=(n, 2), dtype=np.uint64).astype(np.uint32)
    ctr[:3] = [[0, 0, 0, 0], [0xFFFFFFFF] * 4, [7, 0, 0xFFFFFFFF, 1]]
    key[:3] = [[0, 0], [0xFFFFFFFF] * 2, [0xFFFFFFFF, 0]]
    inp = "\n".join(" ".join("%x" % v for v in list(c) + list(k)) for c, k in zip(ctr, key))
    out = subprocess.run([rocrand_philox_exe], input=inp, capture_output=True, text=True, check=True).stdout
    ref = np.array([[int(x, 16) for x in line.split()] for line in out.strip().splitlines()], np.uint32)
    assert ref.shape == (n, 4)
    assert np.array_equal(rng.philox_blocks(ctr, key), ref)


def test_words_layout():
    # element e of a stream = lane e%4 of block e//4 with counter (e//4, tag, tau_lo, tau_hi)
    w = rng.words(0x123456789, 77, (5 << 32) | 9, 10, 3)
    ctr = np.array([[10 + i, 77, 9, 5] for i in range(3)], np.uint32)
    key = np.array([[0x23456789, 0x1]] * 3, np.uint32)
    assert np.array_equal(w, rng.philox_blocks(ctr, key))


def _ulp_err(got, ref_mp):
    out = []
    for g, r in zip(got, ref_mp):
        rf = float(r)
        out.append(abs(mp.mpf(g) - r) / mp.mpf(np.spacing(abs(rf))))
    return max(out)


def test_ln_against_mpmath():
    mp.mp.prec = 120
    rs = np.random.default_rng(2)
    w = rs.integers(0, 2**32, size=3000, dtype=np.uint64)
    w[:6] = [0, 1, 2**31, 2**32 - 1, 0xB504F333, 0x6A09E667]
    u = (w.astype(np.float64) + 0.5) * 2.0**-32
    got = rng.ln(u)
    assert _ulp_err(got, [mp.log(mp.mpf(x)) for x in u]) <= 4


def test_sincos_against_mpmath():
    mp.mp.prec = 120
    rs = np.random.default_rng(3)
    x = rs.random(3000) * (np.pi / 4)
    x[:3] = [1e-9, np.pi / 4, 0.5]
    s, c = rng.sincos_q(x)
    assert _ulp_err(s, [mp.sin(mp.mpf(v)) for v in x]) <= 4
    assert _ulp_err(c, [mp.cos(mp.mpf(v)) for v in x]) <= 4


def test_box_muller_against_textbook():
    """z_a = sqrt(-2 ln u) cos(theta), z_b = ... sin(theta) with the spec's u and theta."""
    mp.mp.prec = 120
    rs = np.random.default_rng(4)
    n = 2000
    wa = rs.integers(0, 2**32, size=n, dtype=np.uint64).astype(np.uint32)
    wb = rs.integers(0, 2**32, size=n, dtype=np.uint64).astype(np.uint32)
    za, zb = rng.box_muller(wa, wb)
    for i in range(n):
        u = (mp.mpf(int(wa[i])) + mp.mpf(0.5)) * mp.mpf(2) ** -32
        R = mp.sqrt(-2 * mp.log(u))
        quad, h = int(wb[i]) >> 30, (int(wb[i]) >> 29) & 1
        f = (mp.mpf(int(wb[i]) & 0x1FFFFFFF) + mp.mpf(0.5)) * mp.mpf(2) ** -29
        phi = f * mp.pi / 4
        psi = (mp.pi / 2 - phi) if h else phi
        th = quad * mp.pi / 2 + psi
        ea, eb = float(R * mp.cos(th)), float(R * mp.sin(th))
        assert abs(za[i] - ea) <= 1e-14 * max(1.0, abs(ea))
        assert abs(zb[i] - eb) <= 1e-14 * max(1.0, abs(eb))


def test_gaussian_stream_statistics():
    z = rng.normal(7, rng.direction_tag(3, 2, 0), 11, 2_000_000)
    n = z.size
    assert abs(z.mean()) < 4 / np.sqrt(n)
    assert abs(z.var() - 1.0) < 4 * np.sqrt(2.0 / n)
    assert stats.kstest(z[:200000], "norm").pvalue > 1e-3
    za, zb = z[0::4], z[1::4]          # the two halves of one Box-Muller pair
    assert abs(np.corrcoef(za, zb)[0, 1]) < 4 / np.sqrt(za.size)
    assert abs(np.corrcoef(za ** 2, zb ** 2)[0, 1]) < 4 / np.sqrt(za.size) * 3
    k = stats.kurtosis(z, fisher=False)
    assert abs(k - 3.0) < 0.02


def test_streams_distinct_by_tag_tau_seed():
    a = rng.normal(0, 1, 0, 64)
    assert not np.array_equal(a, rng.normal(0, 2, 0, 64))
    assert not np.array_equal(a, rng.normal(0, 1, 1, 64))
    assert not np.array_equal(a, rng.normal(1, 1, 0, 64))
    assert np.array_equal(a[10:30], rng.normal(0, 1, 0, 20, first=10))


@pytest.mark.parametrize("r", [2, 4, 64])
def test_factorized_entry_kurtosis_clt(r):
    """entries of G V^T / sqrt(r), G and V iid N(0,1): kurtosis = 3 + 6/r."""
    from oracle import params
    n = 600
    ks = []
    for seed in range(6):
        G = params.factor(seed, 0, 0, 0, 0, n, r)
        V = params.factor(seed, 0, 0, 1, 0, n, r)
        Z = (G @ V.T) / np.sqrt(r)
        ks.append(np.mean(Z ** 4) / np.mean(Z ** 2) ** 2)
    expect = 3.0 + 6.0 / r
    assert abs(np.mean(ks) - expect) < 0.06 * expect
