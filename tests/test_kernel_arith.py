"""CPU checks of the arithmetic identities the gfx950 store kernel relies on.

These do not run the kernel (the GPU parity tests do that); they check, with
exact rational arithmetic, the two short sequences that replace divisions on
the kernel's fast path, so that a change to either is caught without a GPU:

* tile scale: for n = 128 + m (m = the 7 mantissa bits of a bf16 amax),
  S = fma(fma(-q0, 448, n), c, q0) with q0 = n * c, c = RN(1/448), equals
  RN(n / 448); and Y = fma(fma(-S, y0, 1), y0, y0) equals RN(1 / S) for any
  reciprocal estimate y0 within 3 ulp of it.  Scaling by a power of two
  commutes with rounding while the result stays normal, so this gives
  RN(amax / 448) and RN(1 / RN(amax / 448)) for every amax on the fast path.
* quotient: q = x*y, t = fma(q, s, -x), q' = fma(-t, y, q) equals the
  magnitude form copysign(fma(fma(-|x|*y, s, |x|), y, |x|*y), x) bit for bit,
  signed zeros included, and its e4m3 code equals that of the correctly
  rounded quotient RN(x / s) (the OCP e4m3 encoding, round to nearest even).
"""
from fractions import Fraction

import numpy as np
import pytest

from exact_fp import f32_bits as bits, f32_from_bits as from_bits, rn32


def f32(v) -> float:
    """Round a Python float (binary64) to binary32, returned as a float."""
    return float(np.float32(v))


def fma32(a: float, b: float, c: float) -> float:
    """Fused multiply-add in binary32 with IEEE signed-zero rules."""
    exact = Fraction(a) * Fraction(b) + Fraction(c)
    if exact != 0:
        return rn32(exact)
    prod_neg = (np.signbit(a) != np.signbit(b))
    prod_zero = a == 0.0 or b == 0.0
    if prod_zero and c == 0.0:
        return -0.0 if (prod_neg and np.signbit(c)) else 0.0
    return 0.0                                    # exact cancellation: +0 in round-to-nearest


def mul32(a: float, b: float) -> float:
    return f32(a * b)                             # binary64 product of two binary32 is exact


C448 = f32(1.0 / 448.0)


def test_tile_scale_sequence_matches_division():
    for m in range(128):
        n = float(128 + m)
        q0 = mul32(n, C448)
        S = fma32(fma32(-q0, 448.0, n), C448, q0)
        assert bits(S) == bits(rn32(Fraction(128 + m, 448))), m
        y_ref = rn32(1 / Fraction(S))
        for d in range(-3, 4):
            y0 = from_bits(bits(y_ref) + d)
            Y = fma32(fma32(-S, y0, 1.0), y0, y0)
            assert bits(Y) == bits(y_ref), (m, d)


def bf16(u16: int) -> float:
    return from_bits(u16 << 16)


def quotient_sign_free(x: float, s: float, y: float) -> float:
    q = mul32(x, y)
    t = fma32(q, s, -x)
    return fma32(-t, y, q)


def quotient_magnitude(x: float, s: float, y: float) -> float:
    a = abs(x)
    q = mul32(a, y)
    r = fma32(-q, s, a)
    v = fma32(r, y, q)
    return -v if np.signbit(x) else v


def sample_pairs(rng, n):
    """bf16 (amax, x) pairs with |x| <= amax: random, boundaries, zeros."""
    out = []
    amax_bits = list(rng.integers(0x2480, 0x7F80, n // 2)) + [0x3F80, 0x43E0, 0x43E1, 0x7F7F, 0x2480, 0x0080 + 0x2400]
    for ab in amax_bits:
        ab = int(ab)
        a = bf16(ab)
        picks = [ab, ab - 1, 0, 1, 0x0001, int(rng.integers(0, ab + 1)), int(rng.integers(max(0, ab - 0x300), ab + 1))]
        for p in picks:
            if 0 <= p <= ab:
                out.append((a, bf16(p)))
                out.append((a, bf16(p | 0x8000)))     # negative, including -0
    return out


def test_sign_free_quotient_matches_magnitude_form_and_division(orc):
    rng = np.random.default_rng(2024)
    pairs = sample_pairs(rng, 600)
    xs, qs_fast, qs_div = [], [], []
    for amax, x in pairs:
        s = rn32(Fraction(amax) / 448)
        if s < 2.0 ** -64:
            continue                                  # such tiles take the division path
        y = rn32(1 / Fraction(s))
        q1 = quotient_sign_free(x, s, y)
        q2 = quotient_magnitude(x, s, y)
        assert bits(q1) == bits(q2), (amax, x)
        qs_fast.append(q1)
        qs_div.append(f32(np.float32(x) / np.float32(s)))   # IEEE binary32 division
        xs.append(x)
    assert len(xs) > 4000
    codes_fast = orc.e4m3_encode(np.array(qs_fast, np.float32))
    codes_div = orc.e4m3_encode(np.array(qs_div, np.float32))
    assert np.array_equal(codes_fast, codes_div)
    # -0 keeps its sign through the sign-free form (code 0x80)
    assert bits(quotient_sign_free(-0.0, 1.0, 1.0)) == 0x80000000
    assert bits(quotient_sign_free(0.0, 1.0, 1.0)) == 0


@pytest.mark.parametrize("v", [0.5, 1.5, 3.0, 1.0 / 3.0, 1e-30, 3.4e38])
def test_rn32_agrees_with_numpy(v):
    assert bits(rn32(Fraction(v))) == bits(f32(v))
