"""CPU oracle for the quantized skinny-GEMV path (test infrastructure).

Only the test suite, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg
of ``bench.py`` may import this package.  The GPU library (``skinny_gemm_amd``)
never does, and the two share no code: the oracle is ``oracle.c`` compiled by
gcc, loaded here with ctypes, taking and returning numpy arrays.

What each function computes, and the pages' passages it follows, is stated
in ``oracle.c``.  Pins that tie the oracle to something other than itself
live in ``tests/test_oracle_pins.py``.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")

_lib = None


def build(force: bool = False) -> str:
    """Compile ``oracle.c`` into ``liboracle.so`` with gcc (scalar, -O2,
    no contraction, OpenMP)."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp%d" % os.getpid()
        cmd = ["gcc", "-O2", "-std=c11", "-ffp-contract=off", "-fno-fast-math",
               "-fopenmp", "-fPIC", "-shared", "-Wall", "-o", tmp, _SRC, "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB):
        build()
    lib = ctypes.CDLL(_LIB)
    P = ctypes.c_void_p
    I = ctypes.c_int
    lib.oracle_f16_to_double.argtypes = [ctypes.c_uint16]
    lib.oracle_f16_to_double.restype = ctypes.c_double
    lib.oracle_f16_from_double.argtypes = [ctypes.c_double]
    lib.oracle_f16_from_double.restype = ctypes.c_uint16
    lib.oracle_e4m3_to_double.argtypes = [ctypes.c_uint8]
    lib.oracle_e4m3_to_double.restype = ctypes.c_double
    lib.oracle_e2m1_to_double.argtypes = [ctypes.c_uint8]
    lib.oracle_e2m1_to_double.restype = ctypes.c_double
    lib.oracle_quantize_q8_1.argtypes = [P, I, I, P, P, P]
    lib.oracle_quantize_q8_1.restype = None
    lib.oracle_q4_0_blocksums.argtypes = [P, I, I, P, I, P]
    lib.oracle_q4_0_blocksums.restype = None
    lib.oracle_mmvq_q4_0.argtypes = [P, P, I, I, P, P, P, I, P]
    lib.oracle_mmvq_q4_0.restype = None
    lib.oracle_mmvq_q4_k.argtypes = [P, P, I, I, P, P, P, I, P]
    lib.oracle_mmvq_q4_k.restype = None
    lib.oracle_mmvq_q6_k.argtypes = [P, P, P, P, I, I, P, P, I, P]
    lib.oracle_mmvq_q6_k.restype = None
    lib.oracle_mmvq_iq4_xs.argtypes = [P, P, I, I, P, P, I, P]
    lib.oracle_mmvq_iq4_xs.restype = None
    lib.oracle_gemv_nvfp4_w4a16.argtypes = [P, P, ctypes.c_float, I, I, P, I, P, P]
    lib.oracle_gemv_nvfp4_w4a16.restype = None
    lib.oracle_gemv_fp8_w8a16.argtypes = [P, P, I, I, P, I, P, P]
    lib.oracle_gemv_fp8_w8a16.restype = None
    lib.oracle_f16_from_double_array.argtypes = [P, ctypes.c_size_t, P]
    lib.oracle_f16_from_double_array.restype = None
    lib.oracle_num_threads.argtypes = []
    lib.oracle_num_threads.restype = I
    lib.oracle_set_num_threads.argtypes = [I]
    lib.oracle_set_num_threads.restype = None
    _lib = lib
    return lib


def _c(a: np.ndarray, dtype) -> np.ndarray:
    a = np.ascontiguousarray(a)
    if a.dtype != np.dtype(dtype):
        raise TypeError("expected %s, got %s" % (np.dtype(dtype), a.dtype))
    return a


def _p(a: np.ndarray):
    return ctypes.c_void_p(a.ctypes.data)


# ---------------------------------------------------------------- formats

def f16_to_double(bits: int) -> float:
    return _load().oracle_f16_to_double(int(bits))


def f16_from_double(v: float) -> int:
    return int(_load().oracle_f16_from_double(float(v)))


def f16_from_double_array(v: np.ndarray) -> np.ndarray:
    v = _c(np.asarray(v, np.float64).ravel(), np.float64)
    out = np.empty(v.shape, np.uint16)
    _load().oracle_f16_from_double_array(_p(v), v.size, _p(out))
    return out


def e4m3_to_double(b: int) -> float:
    return _load().oracle_e4m3_to_double(int(b))


def e2m1_to_double(c: int) -> float:
    return _load().oracle_e2m1_to_double(int(c))


# ---------------------------------------------------------------- kernels

def quantize_q8_1(x: np.ndarray):
    """x float32 [M][K] -> (qs int8 [M][K], d uint16 [M][K/32], s uint16 [M][K/32])."""
    x = _c(x, np.float32)
    M, K = x.shape
    if K % 32:
        raise ValueError("K must be a multiple of 32")
    qs = np.empty((M, K), np.int8)
    d = np.empty((M, K // 32), np.uint16)
    s = np.empty((M, K // 32), np.uint16)
    _load().oracle_quantize_q8_1(_p(x), M, K, _p(qs), _p(d), _p(s))
    return qs, d, s


def q4_0_blocksums(w_qs: np.ndarray, a_qs: np.ndarray) -> np.ndarray:
    """Integer block dots isum [M][N][K/32] (int32)."""
    w_qs = _c(w_qs, np.uint8)
    a_qs = _c(a_qs, np.int8)
    N, K2 = w_qs.shape
    M, K = a_qs.shape
    assert K == 2 * K2 and K % 32 == 0
    out = np.empty((M, N, K // 32), np.int32)
    _load().oracle_q4_0_blocksums(_p(w_qs), N, K, _p(a_qs), M, _p(out))
    return out


def mmvq_q4_0(w_qs, w_d, a_qs, a_d, a_s) -> np.ndarray:
    """y [M][N] float64."""
    w_qs = _c(w_qs, np.uint8)
    w_d = _c(w_d, np.uint16)
    a_qs = _c(a_qs, np.int8)
    a_d = _c(a_d, np.uint16)
    a_s = _c(a_s, np.uint16)
    N, K2 = w_qs.shape
    M, K = a_qs.shape
    assert K == 2 * K2 and K % 32 == 0
    assert w_d.shape == (N, K // 32) and a_d.shape == (M, K // 32) and a_s.shape == (M, K // 32)
    y = np.empty((M, N), np.float64)
    _load().oracle_mmvq_q4_0(_p(w_qs), _p(w_d), N, K, _p(a_qs), _p(a_d), _p(a_s), M, _p(y))
    return y


def mmvq_q4_k(w_qs, w_hdr, a_qs, a_d, a_s) -> np.ndarray:
    """Q4_K weights (qs [N][K/2], hdr [N][K/256][16]) x Q8_1 -> y [M][N] float64."""
    w_qs = _c(w_qs, np.uint8)
    w_hdr = _c(w_hdr, np.uint8)
    a_qs = _c(a_qs, np.int8)
    a_d = _c(a_d, np.uint16)
    a_s = _c(a_s, np.uint16)
    N, K2 = w_qs.shape
    M, K = a_qs.shape
    assert K == 2 * K2 and K % 256 == 0
    assert w_hdr.shape == (N, K // 256, 16)
    assert a_d.shape == (M, K // 32) and a_s.shape == (M, K // 32)
    y = np.empty((M, N), np.float64)
    _load().oracle_mmvq_q4_k(_p(w_qs), _p(w_hdr), N, K, _p(a_qs), _p(a_d), _p(a_s), M, _p(y))
    return y


def mmvq_q6_k(w_ql, w_qh, w_sc, w_d, a_qs, a_d) -> np.ndarray:
    """Q6_K weights (ql [N][K/2], qh [N][K/4], sc int8 [N][K/16], d [N][K/256])
    x Q8_1 -> y [M][N] float64."""
    w_ql = _c(w_ql, np.uint8)
    w_qh = _c(w_qh, np.uint8)
    w_sc = _c(w_sc, np.int8)
    w_d = _c(w_d, np.uint16)
    a_qs = _c(a_qs, np.int8)
    a_d = _c(a_d, np.uint16)
    N, K2 = w_ql.shape
    M, K = a_qs.shape
    assert K == 2 * K2 and K % 256 == 0
    assert w_qh.shape == (N, K // 4) and w_sc.shape == (N, K // 16) and w_d.shape == (N, K // 256)
    assert a_d.shape == (M, K // 32)
    y = np.empty((M, N), np.float64)
    _load().oracle_mmvq_q6_k(_p(w_ql), _p(w_qh), _p(w_sc), _p(w_d), N, K, _p(a_qs), _p(a_d), M,
                             _p(y))
    return y


def mmvq_iq4_xs(w_qs, w_hdr, a_qs, a_d) -> np.ndarray:
    """IQ4_XS weights (qs [N][K/2], hdr [N][K/256][8]) x Q8_1 (codes and d8)
    -> y [M][N] float64."""
    w_qs = _c(w_qs, np.uint8)
    w_hdr = _c(w_hdr, np.uint8)
    a_qs = _c(a_qs, np.int8)
    a_d = _c(a_d, np.uint16)
    N, K2 = w_qs.shape
    M, K = a_qs.shape
    assert K == 2 * K2 and K % 256 == 0
    assert w_hdr.shape == (N, K // 256, 8)
    assert a_d.shape == (M, K // 32)
    y = np.empty((M, N), np.float64)
    _load().oracle_mmvq_iq4_xs(_p(w_qs), _p(w_hdr), N, K, _p(a_qs), _p(a_d), M, _p(y))
    return y


def gemv_nvfp4_w4a16(codes, scales, g: float, x):
    """-> (y_acc float64 [M][N], y binary16 bits uint16 [M][N])."""
    codes = _c(codes, np.uint8)
    scales = _c(scales, np.uint8)
    x = _c(x, np.uint16)
    N, K2 = codes.shape
    M, K = x.shape
    assert K == 2 * K2 and K % 16 == 0 and scales.shape == (N, K // 16)
    y_acc = np.empty((M, N), np.float64)
    y = np.empty((M, N), np.uint16)
    _load().oracle_gemv_nvfp4_w4a16(_p(codes), _p(scales), float(g), N, K, _p(x), M,
                                    _p(y_acc), _p(y))
    return y_acc, y


def gemv_fp8_w8a16(w, cs, x):
    """-> (y_acc float64 [M][N], y binary16 bits uint16 [M][N])."""
    w = _c(w, np.uint8)
    cs = _c(cs, np.float32)
    x = _c(x, np.uint16)
    N, K = w.shape
    M, K2 = x.shape
    assert K == K2 and cs.shape == (N,)
    y_acc = np.empty((M, N), np.float64)
    y = np.empty((M, N), np.uint16)
    _load().oracle_gemv_fp8_w8a16(_p(w), _p(cs), N, K, _p(x), M, _p(y_acc), _p(y))
    return y_acc, y


def num_threads() -> int:
    return int(_load().oracle_num_threads())


def set_num_threads(n: int) -> None:
    _load().oracle_set_num_threads(int(n))
