"""ctypes front of oracle/philox_normal.c (test infrastructure only).

Streams (the spec of the random numbers the method draws):
  element e of stream (seed, tag, tau) = lane e%4 of Philox4x32-10 with
  counter (e//4, tag, lo32(tau), hi32(tau)) and key (lo32(seed), hi32(seed)),
  Gaussian via the exact-operation Box-Muller transform in the C file.

Tags:
  directions : (layer << 8) | (kind << 1) | factor     factor G=0, V=1
               tau = step t for G, window floor(t/nu) for V
  weights    : (1 << 30) | (slot << 8) | param         slot 0 = global,
               slot l+1 = layer l; tau = 0; seed = model seed
"""
import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "philox_normal.c")
_LIB = os.path.join(_HERE, "_philox_normal.so")
_lib = None


def build(force=False):
    """Compile the C stream with gcc: IEEE binary64, no contraction, no fast-math."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp%d" % os.getpid()
        subprocess.check_call(["gcc", "-O2", "-ffp-contract=off", "-fno-fast-math", "-fopenmp",
                               "-shared", "-fPIC", "-o", tmp, _SRC, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


def lib():
    global _lib
    if _lib is None:
        build()
        L = ctypes.CDLL(_LIB)
        u32p = np.ctypeslib.ndpointer(np.uint32, flags="C")
        f64p = np.ctypeslib.ndpointer(np.float64, flags="C")
        L.oracle_normal_fill.argtypes = [ctypes.c_uint64, ctypes.c_uint32, ctypes.c_uint64,
                                         ctypes.c_int64, ctypes.c_int64, f64p]
        L.oracle_words_fill.argtypes = [ctypes.c_uint64, ctypes.c_uint32, ctypes.c_uint64,
                                        ctypes.c_int64, ctypes.c_int64, u32p]
        L.oracle_ln_array.argtypes = [f64p, f64p, ctypes.c_int64]
        L.oracle_sincos_array.argtypes = [f64p, f64p, f64p, ctypes.c_int64]
        L.oracle_box_muller_array.argtypes = [u32p, u32p, f64p, f64p, ctypes.c_int64]
        L.oracle_philox_array.argtypes = [u32p, u32p, u32p, ctypes.c_int64]
        _lib = L
    return _lib


def philox_blocks(ctr, key):
    """ctr uint32 [n,4], key uint32 [n,2] -> uint32 [n,4]."""
    ctr = np.ascontiguousarray(ctr, np.uint32)
    key = np.ascontiguousarray(key, np.uint32)
    out = np.empty_like(ctr)
    lib().oracle_philox_array(ctr, key, out, ctr.shape[0])
    return out


def words(seed, tag, tau, first_block, n_blocks):
    out = np.empty((n_blocks, 4), np.uint32)
    lib().oracle_words_fill(seed, tag, tau, first_block, n_blocks, out)
    return out


def normal(seed, tag, tau, n, first=0):
    """fp64 standard normals, elements [first, first+n) of the stream."""
    out = np.empty(n, np.float64)
    if n:
        lib().oracle_normal_fill(seed, tag, tau, first, n, out)
    return out


def ln(u):
    u = np.ascontiguousarray(u, np.float64)
    out = np.empty_like(u)
    lib().oracle_ln_array(u, out, u.size)
    return out


def sincos_q(x):
    x = np.ascontiguousarray(x, np.float64)
    s, c = np.empty_like(x), np.empty_like(x)
    lib().oracle_sincos_array(x, s, c, x.size)
    return s, c


def box_muller(wa, wb):
    wa = np.ascontiguousarray(wa, np.uint32)
    wb = np.ascontiguousarray(wb, np.uint32)
    za, zb = np.empty(wa.size), np.empty(wa.size)
    lib().oracle_box_muller_array(wa, wb, za, zb, wa.size)
    return za, zb


# ---- tags -------------------------------------------------------------------
FACTOR_G = 0
FACTOR_V = 1


def direction_tag(layer, kind, factor):
    return (layer << 8) | (kind << 1) | factor


def weight_tag(slot, param):
    return (1 << 30) | (slot << 8) | param
