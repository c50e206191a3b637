"""Exact-arithmetic brute force used to pin the oracle (CPU only).

Nothing here reuses the oracle's code or its float64-then-round shortcut:
every quantity is an exact rational (``fractions.Fraction``) and every
rounding is a search for the nearest representable value, comparing exact
distances, with ties broken towards the even encoding.
"""

from fractions import Fraction

import numpy as np

# The 127 finite non-negative e4m3fn values, listed from the format's
# definition: subnormals m * 2**-9 (m = 0..7) for exponent field 0, then
# (8 + m) * 2**(e - 10) for exponent fields e = 1..15, except e = 15, m = 7
# which is NaN.
E4M3_POS_VALUES = [Fraction(m, 512) for m in range(8)]
for _e in range(1, 16):
    for _m in range(8):
        if _e == 15 and _m == 7:
            continue
        E4M3_POS_VALUES.append(Fraction(8 + _m) * Fraction(2) ** (_e - 10))
assert len(E4M3_POS_VALUES) == 127 and E4M3_POS_VALUES[-1] == 448


def frac_of_f32(v) -> Fraction:
    """Exact value of a float32 (given as np.float32 or a float holding one)."""
    return Fraction(float(np.float32(v)))


def _f32_sign_negative(v) -> bool:
    return bool(np.signbit(np.float32(v)))


def nearest_f32(q: Fraction, negative_zero: bool = False) -> np.float32:
    """Nearest float32 to the exact rational ``q``; ties go to the even significand.

    The search starts from numpy's conversion of ``float(q)`` and examines
    the five float32 values around it, so it only relies on that start being
    within two float32 ulps, never on how numpy or the CPU rounds.
    """
    if q == 0:
        return np.float32(-0.0) if negative_zero else np.float32(0.0)
    start = np.float32(float(q))
    cands = [start]
    lo = hi = start
    for _ in range(2):
        lo = np.nextafter(lo, np.float32(-np.inf), dtype=np.float32)
        hi = np.nextafter(hi, np.float32(np.inf), dtype=np.float32)
        cands += [lo, hi]
    cands = [c for c in cands if np.isfinite(c)]
    best = None
    for c in cands:
        d = abs(Fraction(float(c)) - q)
        bits = int(np.array(c, dtype=np.float32).view(np.uint32))
        key = (d, bits & 1)
        if best is None or key < best[0]:
            best = (key, c)
    (dist, _), choice = best
    # the winner must be strictly inside the window, or the window was too small
    assert choice not in (cands[-1], cands[-2]) or dist == 0
    if choice == 0:
        return np.float32(-0.0) if q < 0 else np.float32(0.0)
    return np.float32(choice)


def nearest_e4m3_code(y: np.float32) -> int:
    """Nearest e4m3fn code to the float32 ``y`` (|y| <= 448), ties to the even code."""
    a = abs(Fraction(float(y)))
    assert a <= 448
    best = min(range(127), key=lambda c: (abs(E4M3_POS_VALUES[c] - a), c & 1))
    return (0x80 if _f32_sign_negative(y) else 0x00) | best


def bf16_frac(bits: int) -> Fraction:
    f = np.array([(bits & 0xFFFF) << 16], dtype=np.uint32).view(np.float32)[0]
    return Fraction(float(f))


def bf16_negative(bits: int) -> bool:
    return bool(bits & 0x8000)


def quantize_tile_exact(bits_list, eps: float):
    """One tile by exact arithmetic: returns (codes, s as np.float32)."""
    vals = [bf16_frac(b) for b in bits_list]
    amax = max((abs(v) for v in vals), default=Fraction(0))
    a = max(amax, frac_of_f32(eps))
    s = nearest_f32(a / 448)
    r = nearest_f32(1 / Fraction(float(s)))
    codes = []
    for b, v in zip(bits_list, vals):
        y = nearest_f32(v * Fraction(float(r)), negative_zero=bf16_negative(b))
        if y > 448:
            y = np.float32(448.0)
        if y < -448:
            y = np.float32(-448.0)
        codes.append(nearest_e4m3_code(y))
    return codes, s


def quantize_exact(bits_2d: np.ndarray, bm: int, bn: int, eps: float):
    """Whole matrix by exact arithmetic (tiny inputs only)."""
    M, N = bits_2d.shape
    TM, TN = -(-M // bm), -(-N // bn)
    q = np.zeros((M, N), dtype=np.uint8)
    s_out = np.zeros((TM, TN), dtype=np.float32)
    for ti in range(TM):
        for tj in range(TN):
            rows = range(ti * bm, min(M, (ti + 1) * bm))
            cols = range(tj * bn, min(N, (tj + 1) * bn))
            idx = [(r, c) for r in rows for c in cols]
            codes, s = quantize_tile_exact([int(bits_2d[r, c]) for r, c in idx], eps)
            for (r, c), code in zip(idx, codes):
                q[r, c] = code
            s_out[ti, tj] = s
    return q, s_out
