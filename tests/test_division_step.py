"""The NVFP4 kernels divide by a per-block divisor d with one shared correctly rounded
reciprocal y = RN(1/d) and one remainder step per quotient:
    q0 = RN(x*y),  r = RN(x - q0*d)  (fma),  q = RN(q0 + r*y)  (fma).
This checks, in exact rational arithmetic, that q equals the correctly rounded
binary32 quotient RN(x/d) on the kernels' operand domain: x a bf16 value, d the
product of an E4M3 scale and a tensor scale amax/2688 with d >= 2^-90 (smaller
divisors take the full division).  Cases are random and adversarial (quotients
within a few ulps of every E2M1 rounding threshold)."""
import random
import struct
from fractions import Fraction

import numpy as np

TWO = Fraction(2)


def rn32(v: Fraction) -> Fraction:
    """Round an exact rational to the nearest binary32 value (ties to even)."""
    if v == 0:
        return Fraction(0)
    sign = -1 if v < 0 else 1
    a = abs(v)
    e = a.numerator.bit_length() - a.denominator.bit_length()
    if TWO ** e > a:
        e -= 1
    e = max(e, -126)
    ulp = TWO ** (e - 23)
    n = a / ulp
    fl = n.numerator // n.denominator
    rem = n - fl
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and fl % 2 == 1):
        fl += 1
    return sign * fl * ulp


def f32(v) -> Fraction:
    return Fraction(float(np.float32(v)))


def bf16(v: float) -> float:
    u = struct.unpack('<I', struct.pack('<f', v))[0]
    u = (u + 0x7FFF + ((u >> 16) & 1)) & 0xFFFF0000
    return struct.unpack('<f', struct.pack('<I', u))[0]


def e4m3_values():
    vals = [(m / 8) * 2.0 ** -6 for m in range(1, 8)]
    vals += [(1 + m / 8) * 2.0 ** (e - 7) for e in range(1, 16) for m in range(8)]
    return [v for v in vals if v <= 448]


def step_quotient(X: Fraction, D: Fraction) -> Fraction:
    y = rn32(1 / D)
    q0 = rn32(X * y)
    r = rn32(X - q0 * D)
    return rn32(q0 + r * y)


def test_remainder_step_is_correctly_rounded_division():
    rng = random.Random(7)
    scales = e4m3_values()
    thresholds = [0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, 6.0, 0.5, 1.0, 2.0, 4.0]
    checked = 0
    for it in range(12000):
        amax = abs(bf16(2.0 ** rng.uniform(-60, 60)))
        if amax == 0.0:
            continue
        S = float(np.float32(amax / 2688.0))
        d = float(np.float32(rng.choice(scales) * S))
        if d < 2.0 ** -90:
            continue
        if it % 2:
            t = rng.choice(thresholds)
            x = bf16(t * d * (1 + rng.choice([-1, 1]) * rng.random() * 2.0 ** -rng.randint(5, 26)))
        else:
            x = bf16(rng.uniform(-amax, amax))
        X, D = f32(x), f32(d)
        assert step_quotient(X, D) == rn32(X / D), (x, d)
        checked += 1
    assert checked > 10000


def test_remainder_step_keeps_the_sign_of_zero():
    """On a zero dividend every step of the remainder form works on zeros and exact
    products, so IEEE's zero-sign rules decide the result; binary64 follows the same rules,
    which lets Python floats model it.  The kernels' form, t = q0*d - x and q = q0 + (-t)*y,
    returns -0 for x = -0 (the quotient's sign, kept by E2M1 as code 0x8); the textbook
    order r = x - q0*d, q = q0 + r*y would return +0 there."""
    import math
    for d in (2.0 ** -90, 0.75, 1.5e35):
        y = 1.0 / d
        for x in (0.0, -0.0):
            q0 = x * y
            t = q0 * d + (-x)          # fma(q0, d, -x): an exact zero
            q = (-t) * y + q0          # fma(-t, y, q0)
            assert q == 0.0 and math.copysign(1.0, q) == math.copysign(1.0, x)
            r = (-q0) * d + x          # fma(-q0, d, x)
            q_textbook = r * y + q0
            assert math.copysign(1.0, q_textbook) == 1.0  # the sign a -0 dividend would lose
