"""Exact brute force for tiny shapes -- TEST INFRASTRUCTURE.

Independent of tq2_oracle.c: binary16 values are decoded by numpy's float16
type (a library routine), sums are exact rationals (fractions.Fraction) and
Python integers, and the only rounding is the final IEEE sequence that the
int8 definition prescribes.  Inputs are the unpacked codes q (integers in
{0,1,2}, shape [N][K]) rather than packed bytes, so this module never reads
the byte layout either.

Page: "BitCPM ternary (1.58-bit)", TQ2_0 definition and block decomposition;
page "gemma4 wNa8o8 requires int8 activations", int8 activation quantizer.
"""
from fractions import Fraction

import numpy as np


def half_exact(bits):
    """Exact rational value of binary16 bit patterns (via numpy float16)."""
    arr = np.asarray(bits, dtype=np.uint16).view(np.float16).astype(np.float64)
    return [Fraction(float(v)) for v in arr.ravel()]


def exact_gemv(q, d_bits, x_bits):
    """y_n = sum_k d_{n,k//256} * (q_nk - 1) * x_k, exactly."""
    q = np.asarray(q, dtype=np.int64)
    N, K = q.shape
    d = np.asarray(d_bits, dtype=np.uint16).reshape(N, K // 256)
    x = half_exact(x_bits)
    out = []
    for n in range(N):
        dn = half_exact(d[n])
        acc = Fraction(0)
        for k in range(K):
            acc += dn[k // 256] * int(q[n, k] - 1) * x[k]
        out.append(acc)
    return out


def exact_gemv_blockwise(q, d_bits, x_bits):
    """The right-hand side of the page's decomposition:
    sum_b d_b * sum_{k in b} x_k (q_k - 1), exactly."""
    q = np.asarray(q, dtype=np.int64)
    N, K = q.shape
    d = np.asarray(d_bits, dtype=np.uint16).reshape(N, K // 256)
    x = half_exact(x_bits)
    out = []
    for n in range(N):
        dn = half_exact(d[n])
        tot = Fraction(0)
        for b in range(K // 256):
            inner = Fraction(0)
            for k in range(b * 256, (b + 1) * 256):
                inner += x[k] * int(q[n, k] - 1)
            tot += dn[b] * inner
        out.append(tot)
    return out


def exact_l1(q, d_bits, x_bits):
    """sum_k |d_{n,b(k)} * x_k| per row, exactly (the tolerance scale)."""
    q = np.asarray(q)
    N, K = q.shape
    d = np.asarray(d_bits, dtype=np.uint16).reshape(N, K // 256)
    x = half_exact(x_bits)
    out = []
    for n in range(N):
        dn = half_exact(d[n])
        out.append(sum(abs(dn[k // 256] * x[k]) for k in range(K)))
    return out


def exact_partials(q, xq):
    """P_nb = sum_{k in b} xq_k (q_nk - 1) with Python integers."""
    q = np.asarray(q, dtype=np.int64)
    N, K = q.shape
    xq = [int(v) for v in np.asarray(xq).ravel()]
    P = [[0] * (K // 256) for _ in range(N)]
    for n in range(N):
        for k in range(K):
            P[n][k // 256] += xq[k] * int(q[n, k] - 1)
    return P


def exact_i8_y(q, d_bits, xq, s):
    """y_n for the int8 path: A_n = sum_b d_b * 2^24 * P_nb must be an
    integer; then y = fl32(fl64(fl64(A) * s) * 2^-24) using Python floats
    (IEEE double, round to nearest even) and numpy.float32."""
    q = np.asarray(q)
    N, K = q.shape
    d = np.asarray(d_bits, dtype=np.uint16).reshape(N, K // 256)
    P = exact_partials(q, xq)
    s64 = float(np.float32(s))
    ys = []
    for n in range(N):
        dn = half_exact(d[n])
        A = sum(dn[b] * (1 << 24) * P[n][b] for b in range(K // 256))
        assert A.denominator == 1
        A = int(A)
        ys.append(np.float32((float(A) * s64) * 2.0 ** -24))
    return np.array(ys, dtype=np.float32)
