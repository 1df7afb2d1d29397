"""Exact rational brute force for tiny Q8_0 problems (test infrastructure).

Independent of ``q8ref.c``: it rebuilds every step with Python's
``fractions.Fraction`` and an IEEE rounding routine written here, so that the
C oracle can be pinned against it:

* ``round_binary(x, p, emin)``: the value nearest to rational x among the
  floating-point numbers with p significant bits and minimum normal exponent
  emin (subnormals below it), ties to even -- the IEEE 754 rounding.
* ``quantize_block_exact``: the Q8_0 block quantiser with each binary32
  operation replaced by its exact result rounded by ``round_binary``.
* ``gemm_exact``: dequantise both operands exactly (d * q as rationals) and
  take the plain matrix product -- the value the blocked form must equal.
"""
import math
import struct
from fractions import Fraction

F32 = (24, -126)     # significand bits, minimum normal exponent
F16 = (11, -14)


def round_binary(x: Fraction, p: int, emin: int, emax: int = None) -> Fraction:
    """Round rational x to the nearest p-bit binary float, ties to even.
    Values beyond emax (if given) return None (overflow)."""
    if x == 0:
        return Fraction(0)
    sign = -1 if x < 0 else 1
    a = abs(x)
    # exponent e with 2^e <= a < 2^(e+1)
    e = a.numerator.bit_length() - a.denominator.bit_length()
    if Fraction(2) ** e > a:
        e -= 1
    e = max(e, emin)                       # subnormal range shares emin's quantum
    quantum = Fraction(2) ** (e - p + 1)
    n = a / quantum                        # want nearest integer to n, ties even
    fl = math.floor(n)
    rem = n - fl
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and fl % 2 == 1):
        fl += 1
    r = fl * quantum
    if emax is not None and r >= Fraction(2) ** (emax + 1):
        return None
    return sign * r


def f32(x: Fraction) -> Fraction:
    return round_binary(Fraction(x), *F32)


def f16_value(bits: int) -> Fraction:
    """Exact value of binary16 bits (finite only)."""
    return Fraction(struct.unpack("<e", struct.pack("<H", bits))[0])


def f16_bits_of(x: Fraction) -> int:
    """binary16 bits of the binary16 value nearest to x (ties even)."""
    r = round_binary(Fraction(x), *F16, emax=15)
    if r is None:
        return 0x7C00 | (0x8000 if x < 0 else 0)
    return struct.unpack("<H", struct.pack("<e", float(r)))[0]


def round_half_away(v: Fraction) -> int:
    s = -1 if v < 0 else 1
    return s * math.floor(abs(v) + Fraction(1, 2))


def quantize_block_exact(x):
    """x: 32 binary32 values (python floats holding binary32 values).
    Returns (q list[int], d16 bits)."""
    xs = [Fraction(float(v)) for v in x]
    amax = max(abs(v) for v in xs)
    d32 = f32(amax / 127)
    if d32 < Fraction(2) ** -126:
        return [0] * 32, 0
    inv = f32(1 / d32)
    q = [round_half_away(f32(v * inv)) for v in xs]
    return q, f16_bits_of(d32)


def gemm_exact(q_a, d_a, q_w, d_w):
    """C[m][n] = sum_k (d_a*q_a)[m][k] * (d_w*q_w)[n][k], exact rationals.
    q_*: nested lists / int arrays [rows][K]; d_*: binary16 bits [rows][K/32]."""
    M, K = len(q_a), len(q_a[0])
    N = len(q_w)
    da = [[f16_value(int(b)) for b in row] for row in d_a]
    dw = [[f16_value(int(b)) for b in row] for row in d_w]
    A = [[da[m][k // 32] * int(q_a[m][k]) for k in range(K)] for m in range(M)]
    W = [[dw[n][k // 32] * int(q_w[n][k]) for k in range(K)] for n in range(N)]
    return [[sum(A[m][k] * W[n][k] for k in range(K)) for n in range(N)] for m in range(M)]
