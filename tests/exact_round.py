"""Exact round-to-nearest-even of rational numbers into binary floating-point
formats, in plain integer arithmetic (Python Fractions).  The tests use it as
an independent reference for the oracle's rounding helpers: it shares no code
with them and takes no float intermediate.

A format is (p, emin, emax): p significant bits, normal binades 2^emin ..
2^emax, subnormals below 2^emin with spacing 2^(emin - p + 1), and overflow to
infinity for results at or beyond 2^(emax + 1).
"""

from fractions import Fraction
import math

BF16 = (8, -126, 127)
F32 = (24, -126, 127)
F16 = (11, -14, 15)


def _floor_log2(a):
    """floor(log2(a)) of a positive Fraction, exactly."""
    e = a.numerator.bit_length() - a.denominator.bit_length()
    # 2^e <= a < 2^(e+1) after at most one correction either way
    while Fraction(2) ** e > a:
        e -= 1
    while Fraction(2) ** (e + 1) <= a:
        e += 1
    return e


def _round_half_even(n):
    """Nearest integer to the Fraction n, ties to even."""
    fl = math.floor(n)
    rem = n - fl
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and fl % 2 == 1):
        fl += 1
    return fl


def rne(q, fmt):
    """The value of format fmt nearest to the Fraction q (ties to even), as a
    Fraction, or +-math.inf on overflow."""
    p, emin, emax = fmt
    q = Fraction(q)
    if q == 0:
        return Fraction(0)
    s = -1 if q < 0 else 1
    a = abs(q)
    e = max(_floor_log2(a), emin)
    ulp = Fraction(2) ** (e - p + 1)
    r = _round_half_even(a / ulp) * ulp
    if r >= Fraction(2) ** (emax + 1):
        return s * math.inf
    return s * r


def rne_sqrt_ratio(h, S, fmt):
    """RNE of h / sqrt(S) for a Fraction h and a positive Fraction S, decided
    exactly: v >= c  <=>  h^2 >= c^2 S  for v, c >= 0 (no square root is
    taken).  Returns (value as Fraction, tie_distance) where tie_distance is
    the distance of v from the nearest rounding midpoint in ulps, estimated
    in float (to tell how close the exact value came to a boundary)."""
    p, emin, emax = fmt
    h = Fraction(h)
    S = Fraction(S)
    if h == 0:
        return Fraction(0), 1.0
    s = -1 if h < 0 else 1
    a2 = h * h  # |v|^2 * S
    est = abs(float(h)) / math.sqrt(float(S))

    def le(c):  # c <= |v| for c >= 0
        return c * c * S <= a2

    e = max(math.frexp(est)[1] - 1, emin)
    for _ in range(4):
        ulp = Fraction(2) ** (e - p + 1)
        n = int(est / float(ulp))
        while not le(n * ulp):
            n -= 1
        while le((n + 1) * ulp):
            n += 1
        # n * ulp <= |v| < (n + 1) * ulp; fix the binade if the estimate was off
        if n >= 2 ** p and e < emax + 1:
            e += 1
            continue
        if n < 2 ** (p - 1) and e > emin:
            e -= 1
            continue
        break
    mid = (n + Fraction(1, 2)) * ulp
    if mid * mid * S < a2:
        n += 1
    elif mid * mid * S == a2:
        n += n % 2
    r = n * ulp
    t = est / float(ulp)
    tie_dist = abs((t - math.floor(t)) - 0.5)
    if r >= Fraction(2) ** (emax + 1):
        return s * math.inf, tie_dist
    return s * r, tie_dist
