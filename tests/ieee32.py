"""Exact IEEE-754 binary32 reference arithmetic for the tests.

Results are computed as exact rationals (fractions.Fraction) and rounded to
binary32 by round-to-nearest, ties-to-even, written here from the IEEE-754
definition: the representable numbers are m * 2**(e - 23) with 2**23 <= m < 2**24
for normal numbers (e in -126..127) and m < 2**23 at e = -126 for subnormals.
Any NaN result is reported as the canonical pattern 0x7FFFFFFF, the simulator's
convention for arithmetic results.
"""
from fractions import Fraction

CANON_NAN = 0x7FFFFFFF
INF_BITS = 0x7F800000


def classify(bits):
    sign = bits >> 31
    exp = (bits >> 23) & 0xFF
    frac = bits & 0x7FFFFF
    if exp == 0xFF:
        return ("nan", sign, None) if frac else ("inf", sign, None)
    if exp == 0:
        val = Fraction(frac, 1 << 149)
    else:
        val = Fraction((1 << 23) | frac) * Fraction(2) ** (exp - 150)
    return ("num", sign, -val if sign else val)


def _floor_log2(x: Fraction) -> int:
    # largest e with 2**e <= x, for x > 0
    n, d = x.numerator, x.denominator
    e = n.bit_length() - d.bit_length()
    if Fraction(2) ** e > x:
        e -= 1
    elif Fraction(2) ** (e + 1) <= x:
        e += 1
    return e


def round_f32(x: Fraction, zero_sign: int = 0) -> int:
    """Round an exact rational to binary32 bits (RNE).  zero_sign gives the sign
    of an exact zero result."""
    if x == 0:
        return zero_sign << 31
    sign = 1 if x < 0 else 0
    a = -x if sign else x
    e = max(_floor_log2(a), -126)
    q = Fraction(2) ** (e - 23)          # quantum at this binade
    m = a / q
    mi = m.numerator // m.denominator
    rem = m - mi
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and (mi & 1)):
        mi += 1
    if mi == 1 << 24:                    # carried into the next binade
        mi = 1 << 23
        e += 1
    if e > 127:
        return (sign << 31) | INF_BITS
    if mi < (1 << 23):                   # subnormal (or rounded to zero)
        return (sign << 31) | mi
    return (sign << 31) | ((e + 127) << 23) | (mi - (1 << 23))


def _special(kind_a, kind_b):
    return kind_a == "nan" or kind_b == "nan"


def add(a_bits, b_bits, negate_b=False):
    ka, sa, va = classify(a_bits)
    kb, sb, vb = classify(b_bits)
    if negate_b:
        sb ^= 1
        vb = -vb if vb is not None else None
    if _special(ka, kb):
        return CANON_NAN
    if ka == "inf" and kb == "inf":
        return CANON_NAN if sa != sb else (sa << 31) | INF_BITS
    if ka == "inf":
        return (sa << 31) | INF_BITS
    if kb == "inf":
        return (sb << 31) | INF_BITS
    s = va + vb
    if s == 0:
        zs = sa if (va == 0 and vb == 0 and sa == sb) else 0
        return round_f32(s, zs)
    return round_f32(s)


def sub(a_bits, b_bits):
    return add(a_bits, b_bits, negate_b=True)


def mul(a_bits, b_bits):
    ka, sa, va = classify(a_bits)
    kb, sb, vb = classify(b_bits)
    if _special(ka, kb):
        return CANON_NAN
    sign = sa ^ sb
    if ka == "inf" or kb == "inf":
        other = vb if ka == "inf" else va
        if other is not None and other == 0:
            return CANON_NAN
        return (sign << 31) | INF_BITS
    p = va * vb
    return round_f32(p, sign)


def fma(a_bits, b_bits, c_bits):
    ka, sa, va = classify(a_bits)
    kb, sb, vb = classify(b_bits)
    kc, sc, vc = classify(c_bits)
    if ka == "nan" or kb == "nan" or kc == "nan":
        return CANON_NAN
    ps = sa ^ sb
    if ka == "inf" or kb == "inf":
        other = vb if ka == "inf" else va
        if other is not None and other == 0:
            return CANON_NAN
        if kc == "inf" and sc != ps:
            return CANON_NAN
        return (ps << 31) | INF_BITS
    if kc == "inf":
        return (sc << 31) | INF_BITS
    p = va * vb
    s = p + vc
    if s == 0:
        zs = ps if (p == 0 and vc == 0 and ps == sc) else 0
        return round_f32(s, zs)
    return round_f32(s)
