"""Exact binary32 rounding for the CPU pins (independent of the oracle and the kernels).

Two routes to the correctly rounded binary32 value of a quotient, written from
the IEEE 754 definition (round to nearest, ties to even, subnormals kept):

* ``rn32(Fraction)`` rounds an exact rational: slow, obviously correct, used
  for the tile scales (a few thousand values) and to check the fast route;
* ``rn32_div(a, b)`` rounds a / b for binary32 arrays with integer arithmetic
  only: both significands are normalized to 24-bit integers, the quotient of
  the significands is taken to 26-27 bits with its remainder as a sticky bit,
  and the kept bits are rounded at the binary32 quantum of the result's binade
  (2^-149 in the subnormal range).

Neither calls a floating-point division.
"""
from fractions import Fraction
import struct

import numpy as np


def f32_bits(v: float) -> int:
    return struct.unpack("<I", struct.pack("<f", v))[0]


def f32_from_bits(u: int) -> float:
    return struct.unpack("<f", struct.pack("<I", u & 0xFFFFFFFF))[0]


def rn32(x: Fraction) -> float:
    """Exact rational -> binary32, round to nearest, ties to even (finite range)."""
    if x == 0:
        return 0.0
    neg = x < 0
    m = -x if neg else x
    e = m.numerator.bit_length() - m.denominator.bit_length()
    if Fraction(2) ** e > m:
        e -= 1
    while Fraction(2) ** (e + 1) <= m:
        e += 1
    q_exp = max(e, -126) - 23                     # quantum of the binade (subnormals: 2^-149)
    quantum = Fraction(2) ** q_exp
    n, rem = divmod(m, quantum)                   # n integer part, rem in [0, quantum)
    n = int(n)
    if rem * 2 > quantum or (rem * 2 == quantum and n % 2 == 1):
        n += 1
    v = float(n * quantum)                        # exact in binary64
    assert v < 2.0 ** 128, "overflow"
    return -v if neg else v


def _significand(v):
    """Positive finite nonzero binary32 array -> (M, e) with v = M * 2^e, M in [2^23, 2^24)."""
    u = np.ascontiguousarray(v, dtype=np.float32).view(np.uint32).astype(np.int64)
    exp = (u >> 23) & 0xFF
    man = u & 0x7FFFFF
    M = np.where(exp > 0, man | 0x800000, man)
    e = np.where(exp > 0, exp - 150, -149)
    # subnormals: shift the significand up to 24 bits
    nbits = np.frexp(M.astype(np.float64))[1].astype(np.int64)   # bit length (M < 2^24: exact)
    sh = 24 - nbits
    return M << sh, e - sh


def rn32_div(a, b):
    """RN32(a / b) elementwise for binary32 arrays: a finite, b finite and > 0."""
    a = np.ascontiguousarray(a, dtype=np.float32)
    b = np.broadcast_to(np.asarray(b, dtype=np.float32), a.shape)
    assert np.all(np.isfinite(a)) and np.all(np.isfinite(b)) and np.all(b > 0)
    neg = np.signbit(a)
    mag = np.abs(a)
    zero = mag == 0
    A, ea = _significand(np.where(zero, b, mag))     # zeros: any finite quotient, replaced below
    B, eb = _significand(b)
    num = A << 26                                  # < 2^50
    N = num // B                                   # in (2^25, 2^27)
    rem = num - N * B
    base = ea - eb - 26                            # a / b = (N + rem / B) * 2^base
    nb = np.frexp(N.astype(np.float64))[1].astype(np.int64)     # bit length of N (exact: N < 2^53)
    E = nb - 1 + base                              # floor(log2(a / b))
    qe = np.maximum(E, -126) - 23                  # binary32 quantum exponent
    shift = np.minimum(qe - base, 62)              # >= 2; beyond 62 everything rounds to 0
    keep = N >> shift
    dropped = N & ((np.int64(1) << shift) - 1)
    half = np.int64(1) << (shift - 1)
    up = (dropped > half) | ((dropped == half) & ((rem != 0) | ((keep & 1) == 1)))
    keep = keep + up
    out = np.ldexp(keep.astype(np.float64), qe.astype(np.int32))   # keep <= 2^24: exact
    assert np.all(out < 2.0 ** 128), "quotient overflows binary32"
    out = np.where(zero, 0.0, out).astype(np.float32)
    return np.where(neg, -out, out).astype(np.float32)
