"""CPU oracle for the TQ2_0 ternary decode matvec -- TEST INFRASTRUCTURE.

Only the tests, the smoke check and the benchmark's CPU-baseline leg may
import this package.  It shares no code with the GPU library: it parses the
byte layout with its own C code (tq2_oracle.c) and takes numpy arrays.

Functions (each cites its passage in tq2_oracle.c):
  pack(W)                      -> codes, scales, bad_blocks
  dequant(codes, scales, N, K) -> W
  gemv(codes, scales, N, K, x_bits) -> y (fp32, fp64 accumulation)
  quantize_i8(x_bits, s)       -> x_q
  partials_i8(codes, N, K, x_q) -> P [N][K/256]
  gemv_i8q(codes, scales, N, K, x_q, s) -> y, P
  gemv_i8(codes, scales, N, K, x_bits, s) -> y
  requant_i8(y, s_out)         -> y_q, y_deq
  silu_mul(g, u)               -> h (fp64)
  gemm(codes, scales, N, K, X_bits[M][K]) -> Y[M][N] (one matvec per token)
  gemm_i8q(codes, scales, N, K, XQ[M][K], s) -> Y[M][N] (one int8 matvec per token)
  half_to_float(bits), float_to_half(value)
  threads(), set_threads(n)
"""
import ctypes
import os

import numpy as np

from . import build as _build

_LIB = None


def _lib():
    global _LIB
    if _LIB is None:
        # TQ2_ORACLE_SANITIZED=1 loads the AddressSanitizer/UBSan build
        # (the process must preload the sanitizer runtime)
        san = os.environ.get("TQ2_ORACLE_SANITIZED") == "1"
        path = _build.SAN_LIB if san else _build.LIB
        if not os.path.exists(path):
            _build.build(sanitize=san)
        lib = ctypes.CDLL(path)
        P = ctypes.c_void_p
        I64 = ctypes.c_int64
        lib.oracle_half_to_float.argtypes = [ctypes.c_uint16]
        lib.oracle_half_to_float.restype = ctypes.c_float
        lib.oracle_float_to_half.argtypes = [ctypes.c_float]
        lib.oracle_float_to_half.restype = ctypes.c_uint16
        lib.oracle_pack.argtypes = [P, I64, I64, P, P]
        lib.oracle_pack.restype = I64
        lib.oracle_dequant.argtypes = [P, P, I64, I64, P]
        lib.oracle_dequant.restype = None
        lib.oracle_gemv.argtypes = [P, P, I64, I64, P, P]
        lib.oracle_gemv.restype = None
        lib.oracle_quantize_i8.argtypes = [P, I64, ctypes.c_float, P]
        lib.oracle_quantize_i8.restype = None
        lib.oracle_partials_i8.argtypes = [P, I64, I64, P, P]
        lib.oracle_partials_i8.restype = None
        lib.oracle_gemv_i8q.argtypes = [P, P, I64, I64, P, ctypes.c_float, P, P]
        lib.oracle_gemv_i8q.restype = None
        lib.oracle_gemv_i8.argtypes = [P, P, I64, I64, P, ctypes.c_float, P]
        lib.oracle_gemv_i8.restype = None
        lib.oracle_requant_i8.argtypes = [P, I64, ctypes.c_float, P, P]
        lib.oracle_requant_i8.restype = None
        lib.oracle_silu_mul.argtypes = [P, P, I64, P]
        lib.oracle_silu_mul.restype = None
        lib.oracle_gemm.argtypes = [P, P, I64, I64, P, I64, P]
        lib.oracle_gemm.restype = None
        lib.oracle_threads.argtypes = []
        lib.oracle_threads.restype = ctypes.c_int
        lib.oracle_set_threads.argtypes = [ctypes.c_int]
        lib.oracle_set_threads.restype = None
        _LIB = lib
    return _LIB


def _c(a, dtype):
    a = np.ascontiguousarray(a, dtype=dtype)
    return a, a.ctypes.data_as(ctypes.c_void_p)


def _shape_check(N, K):
    if N < 1 or K < 256 or K % 256:
        raise ValueError(f"bad shape N={N} K={K}")


def threads() -> int:
    """Threads the oracle's row loops use (OpenMP)."""
    return int(_lib().oracle_threads())


def set_threads(n: int) -> None:
    """Threads for the oracle's row loops from now on (OpenMP)."""
    _lib().oracle_set_threads(int(n))


def half_to_float(bits: int) -> float:
    return float(_lib().oracle_half_to_float(int(bits)))


def float_to_half(value: float) -> int:
    return int(_lib().oracle_float_to_half(float(value)))


def pack(W):
    W, pW = _c(W, np.float32)
    N, K = W.shape
    _shape_check(N, K)
    codes = np.zeros((N, K // 4), np.uint8)
    scales = np.zeros((N, K // 256), np.uint16)
    bad = _lib().oracle_pack(pW, N, K, codes.ctypes.data_as(ctypes.c_void_p),
                             scales.ctypes.data_as(ctypes.c_void_p))
    return codes, scales, int(bad)


def dequant(codes, scales, N, K):
    _shape_check(N, K)
    codes, pc = _c(codes, np.uint8)
    scales, ps = _c(scales, np.uint16)
    assert codes.size == N * K // 4 and scales.size == N * K // 256
    W = np.empty((N, K), np.float32)
    _lib().oracle_dequant(pc, ps, N, K, W.ctypes.data_as(ctypes.c_void_p))
    return W


def gemv(codes, scales, N, K, x_bits):
    _shape_check(N, K)
    codes, pc = _c(codes, np.uint8)
    scales, ps = _c(scales, np.uint16)
    x_bits, px = _c(x_bits, np.uint16)
    assert codes.size == N * K // 4 and scales.size == N * K // 256 and x_bits.size == K
    y = np.empty(N, np.float32)
    _lib().oracle_gemv(pc, ps, N, K, px, y.ctypes.data_as(ctypes.c_void_p))
    return y


def quantize_i8(x_bits, s):
    x_bits, px = _c(x_bits, np.uint16)
    K = x_bits.size
    xq = np.empty(K, np.int8)
    _lib().oracle_quantize_i8(px, K, float(np.float32(s)), xq.ctypes.data_as(ctypes.c_void_p))
    return xq


def partials_i8(codes, N, K, xq):
    _shape_check(N, K)
    codes, pc = _c(codes, np.uint8)
    xq, pq = _c(xq, np.int8)
    P = np.empty((N, K // 256), np.int32)
    _lib().oracle_partials_i8(pc, N, K, pq, P.ctypes.data_as(ctypes.c_void_p))
    return P


def gemv_i8q(codes, scales, N, K, xq, s):
    _shape_check(N, K)
    codes, pc = _c(codes, np.uint8)
    scales, ps = _c(scales, np.uint16)
    xq, pq = _c(xq, np.int8)
    y = np.empty(N, np.float32)
    P = np.empty((N, K // 256), np.int32)
    _lib().oracle_gemv_i8q(pc, ps, N, K, pq, float(np.float32(s)),
                           y.ctypes.data_as(ctypes.c_void_p), P.ctypes.data_as(ctypes.c_void_p))
    return y, P


def gemv_i8(codes, scales, N, K, x_bits, s):
    _shape_check(N, K)
    codes, pc = _c(codes, np.uint8)
    scales, ps = _c(scales, np.uint16)
    x_bits, px = _c(x_bits, np.uint16)
    y = np.empty(N, np.float32)
    _lib().oracle_gemv_i8(pc, ps, N, K, px, float(np.float32(s)), y.ctypes.data_as(ctypes.c_void_p))
    return y


def requant_i8(y, s_out):
    y, py = _c(y, np.float32)
    N = y.size
    yq = np.empty(N, np.int8)
    yd = np.empty(N, np.float32)
    _lib().oracle_requant_i8(py, N, float(np.float32(s_out)), yq.ctypes.data_as(ctypes.c_void_p),
                             yd.ctypes.data_as(ctypes.c_void_p))
    return yq, yd


def silu_mul(g, u):
    g, pg = _c(g, np.float32)
    u, pu = _c(u, np.float32)
    h = np.empty(g.size, np.float64)
    _lib().oracle_silu_mul(pg, pu, g.size, h.ctypes.data_as(ctypes.c_void_p))
    return h


def gemm(codes, scales, N, K, X_bits):
    _shape_check(N, K)
    codes, pc = _c(codes, np.uint8)
    scales, ps = _c(scales, np.uint16)
    X_bits, px = _c(X_bits, np.uint16)
    M = X_bits.size // K
    assert X_bits.size == M * K and M >= 1
    Y = np.empty((M, N), np.float32)
    _lib().oracle_gemm(pc, ps, N, K, px, M, Y.ctypes.data_as(ctypes.c_void_p))
    return Y


def gemm_i8q(codes, scales, N, K, XQ, s):
    """The int8 matvec (gemv_i8q: page "gemma4 wNa8o8 requires int8
    activations", Implemented section) for each of M tokens of pre-quantized
    activations XQ[M][K] sharing the activation scale s; Y[M][N] fp32."""
    _shape_check(N, K)
    XQ = np.ascontiguousarray(XQ, np.int8)
    M = XQ.size // K
    assert XQ.size == M * K and M >= 1
    return np.stack([gemv_i8q(codes, scales, N, K, XQ.reshape(M, K)[m], s)[0] for m in range(M)])

