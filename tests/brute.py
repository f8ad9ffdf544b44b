"""Pure-Python brute force for tiny inputs: exact rationals, no numpy arithmetic.

Used only to pin the float64 oracle.  bf16 bits are decoded bit by bit from the IEEE-754
layout (sign, 8-bit exponent with bias 127, 7-bit fraction), every sum and product is an
exact ``fractions.Fraction``, and the one square root of RMSNorm is taken in ``decimal``
with 60 significant digits.
"""

from decimal import Decimal, getcontext
from fractions import Fraction


def bf16_value(bits: int) -> Fraction:
    """Exact rational value of a finite bf16 bit pattern."""
    bits = int(bits) & 0xFFFF
    sign = -1 if bits >> 15 else 1
    exp = (bits >> 7) & 0xFF
    frac = bits & 0x7F
    if exp == 0xFF:
        raise ValueError("inf/nan has no rational value")
    if exp == 0:  # subnormal: 0.frac * 2**-126
        return sign * Fraction(frac, 1 << 7) * Fraction(1, 1 << 126)
    mant = Fraction(128 + frac, 128)
    e = exp - 127
    return sign * mant * (Fraction(1 << e) if e >= 0 else Fraction(1, 1 << -e))


def matrix(bits_2d):
    return [[bf16_value(b) for b in row] for row in bits_2d]


def gather(shards):
    """Rows of shard 0, then shard 1, ... (sequence all-gather, rank-major)."""
    out = []
    for s in shards:
        out.extend([list(r) for r in s])
    return out


def matmul(a, b):
    n_in = len(b)
    n_out = len(b[0])
    return [[sum((row[k] * b[k][j] for k in range(n_in)), Fraction(0)) for j in range(n_out)]
            for row in a]


def add(a, b):
    return [[x + y for x, y in zip(ra, rb)] for ra, rb in zip(a, b)]


def rmsnorm_row(h_row, gamma, eps):
    """h / sqrt(mean(h^2) + eps) * gamma with an exact mean and a 60-digit square root."""
    getcontext().prec = 60
    ms = sum((x * x for x in h_row), Fraction(0)) / len(h_row) + Fraction(eps)
    root = (Decimal(ms.numerator) / Decimal(ms.denominator)).sqrt()
    return [float(Decimal(x.numerator) / Decimal(x.denominator) / root
                  * (Decimal(g.numerator) / Decimal(g.denominator)))
            for x, g in zip(h_row, gamma)]


def round_bf16(x: Fraction) -> Fraction:
    """Round a rational to the nearest value with 8 significant bits, ties to even."""
    x = Fraction(x)
    if x == 0:
        return Fraction(0)
    sign = -1 if x < 0 else 1
    a = abs(x)
    e = a.numerator.bit_length() - a.denominator.bit_length()
    if Fraction(2) ** e > a:
        e -= 1
    while Fraction(2) ** (e + 1) <= a:
        e += 1
    scaled = a / Fraction(2) ** (e - 7)          # in [128, 256)
    n = scaled.numerator // scaled.denominator
    rem = scaled - n
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and n % 2 == 1):
        n += 1
    return sign * n * Fraction(2) ** (e - 7)


def bf16_bits(x: Fraction) -> int:
    """Storage bits of the bf16 value nearest to ``x`` (ties to even), built field by field:
    sign bit, 8-bit biased exponent, 7-bit fraction.  Normal range and zero only."""
    r = round_bf16(Fraction(x))
    if r == 0:
        return 0x8000 if Fraction(x) < 0 else 0
    sign = 1 if r < 0 else 0
    a = abs(r)
    e = 0
    while Fraction(2) ** (e + 1) <= a:
        e += 1
    while Fraction(2) ** e > a:
        e -= 1
    if not -126 <= e <= 127:
        raise ValueError("outside the normal bf16 range")
    frac = (a / Fraction(2) ** e - 1) * 128      # exact: r has 8 significant bits
    assert frac.denominator == 1
    return (sign << 15) | ((e + 127) << 7) | int(frac)
