"""Plain definitions for the floating-point front and back end of the exact
product: an enclosure (lo, hi) of A @ B in exact real arithmetic.

TEST INFRASTRUCTURE ONLY: imported by the test suite, the smoke check and the
``cpu_baseline`` leg of ``bench.py``; never by the product path.

Follows the page "enclosure-gemm":

* "Method": operands are scaled by a power of two and floored into
  two's-complement integers; where the scaling is lossless the integer inner
  product is the real inner product.  The exact integer S with its binary
  exponent Q is rounded outward once: lo is the largest format value not above
  S * 2^-Q, hi the smallest not below it, and lo == hi exactly when S * 2^-Q
  is representable.  Overflow saturates to the largest finite value inward and
  to infinity outward.
* "Requirements and limits": K <= 2^17; the capacity budget comes from the
  335-bit product of the primes below 256; non-finite operands are rejected.
* "Correctness": the reference is exact rational arithmetic (every binary64
  value is a rational); with lossless scaling the pair equals the exact floor
  and ceiling in the format.

Readings taken where the page is silent:
  * the scale of an operand is its coarsest lossless one: F = -(the smallest
    exponent of a lowest set bit over its nonzero entries), F = 0 for an
    all-zero operand.  Every lossless scale gives the same exact product, and
    the coarsest needs the fewest bits (so the fewest primes);
  * an exact-zero entry of the product gives (+0.0, +0.0);
  * binary32 operands are exact binary64 values; their pair is rounded in
    binary32.

Parity is pinned in tests/test_oracle_enclose.py: directed rounding against
math.nextafter / numpy.nextafter and exactly representable values, overflow
and the subnormal boundary by their definitions, integer operands against an
int64 product, and the scaled-integer product against a brute-force Fraction
sum.
"""
from __future__ import annotations

import math
from fractions import Fraction
from typing import Dict, Tuple

import numpy as np

# precision p (significand bits, hidden bit included), emin, emax
FORMATS: Dict[str, Tuple[int, int, int]] = {
    "binary64": (53, -1022, 1023),
    "binary32": (24, -126, 127),
}


def exact(x: float) -> Fraction:
    """The rational value of a finite binary64 number (enclosure-gemm, "Correctness")."""
    n, d = float(x).as_integer_ratio()
    return Fraction(n, d)


def _max_finite(fmt: str) -> Fraction:
    p, _, emax = FORMATS[fmt]
    return (2 - Fraction(1, 2 ** (p - 1))) * Fraction(2) ** emax


def _floor_log2(v: Fraction) -> int:
    """E with 2^E <= v < 2^(E+1), for v > 0."""
    E = v.numerator.bit_length() - v.denominator.bit_length()
    if Fraction(2) ** E > v:
        E -= 1
    return E


def _down_positive(v: Fraction, fmt: str) -> Fraction:
    """Largest format value <= v, for v > 0 (may be 0, never +inf)."""
    p, emin, emax = FORMATS[fmt]
    E = _floor_log2(v)
    if E > emax:
        return _max_finite(fmt)
    u = Fraction(2) ** (max(E, emin) - p + 1)       # the grid step at v
    return math.floor(v / u) * u


def _up_positive(v: Fraction, fmt: str):
    """Smallest format value >= v, for v > 0 (a Fraction, or math.inf)."""
    p, emin, emax = FORMATS[fmt]
    E = _floor_log2(v)
    if E > emax:
        return math.inf
    u = Fraction(2) ** (max(E, emin) - p + 1)
    r = math.ceil(v / u) * u
    return math.inf if r > _max_finite(fmt) else r


def _to_float(r) -> float:
    # r lies on the format's grid (or is inf): the conversion is exact
    return r if isinstance(r, float) else float(r)


def round_down(v: Fraction, fmt: str = "binary64") -> float:
    """The largest value of the format not above v."""
    if v == 0:
        return 0.0
    if v > 0:
        return _to_float(_down_positive(v, fmt))
    return -_to_float(_up_positive(-v, fmt))


def round_up(v: Fraction, fmt: str = "binary64") -> float:
    """The smallest value of the format not below v."""
    if v == 0:
        return 0.0
    if v > 0:
        return _to_float(_up_positive(v, fmt))
    return -_to_float(_down_positive(-v, fmt))


def lowest_set_bit_exponent(x: float) -> int:
    """t with x = odd * 2^t, for finite nonzero x."""
    n, d = float(x).as_integer_ratio()
    if d > 1:
        return -(d.bit_length() - 1)      # d is a power of two, n odd
    return (n & -n).bit_length() - 1


def coarsest_lossless_scale(X: np.ndarray) -> int:
    """F such that every x * 2^F is an integer and some entry is odd (0 if X == 0)."""
    vals = [float(x) for x in np.asarray(X, dtype=np.float64).ravel() if x != 0]
    if not vals:
        return 0
    if not all(math.isfinite(v) for v in vals):
        raise ValueError("non-finite operand")
    return -min(lowest_set_bit_exponent(v) for v in vals)


def scaled_integers(X: np.ndarray, F: int) -> np.ndarray:
    """floor(x * 2^F) for every entry, as Python integers (object array)."""
    X = np.asarray(X, dtype=np.float64)
    out = np.empty(X.shape, dtype=object)
    for idx, x in np.ndenumerate(X):
        out[idx] = math.floor(exact(x) * Fraction(2) ** F)
    return out


def product_exact_fractions(A: np.ndarray, B: np.ndarray) -> np.ndarray:
    """sum_k A[i,k] * B[k,j] in exact rationals, term by term (brute force)."""
    A = np.asarray(A, dtype=np.float64)
    B = np.asarray(B, dtype=np.float64)
    M, K = A.shape
    N = B.shape[1]
    out = np.empty((M, N), dtype=object)
    for i in range(M):
        for j in range(N):
            s = Fraction(0)
            for k in range(K):
                s += exact(A[i, k]) * exact(B[k, j])
            out[i, j] = s
    return out


def product_exact_scaled(A: np.ndarray, B: np.ndarray) -> Tuple[np.ndarray, int]:
    """(S, Q) with A @ B == S * 2^-Q exactly: the page's lossless scaling of
    each operand to integers, then one integer product."""
    Fa = coarsest_lossless_scale(A)
    Fb = coarsest_lossless_scale(B)
    Ai = scaled_integers(A, Fa)
    Bi = scaled_integers(B, Fb)
    return Ai.dot(Bi), Fa + Fb


def enclose_from_integer(S: np.ndarray, Q: int, fmt: str = "binary64") -> Tuple[np.ndarray, np.ndarray]:
    """(lo, hi) of S * 2^-Q entrywise, outward rounded once."""
    S = np.asarray(S, dtype=object)
    dt = np.float64 if fmt == "binary64" else np.float32
    lo = np.empty(S.shape, dtype=dt)
    hi = np.empty(S.shape, dtype=dt)
    scale = Fraction(1, 2 ** Q) if Q >= 0 else Fraction(2 ** -Q)
    for idx, s in np.ndenumerate(S):
        v = Fraction(int(s)) * scale
        lo[idx] = round_down(v, fmt)
        hi[idx] = round_up(v, fmt)
    return lo, hi


def enclose(A: np.ndarray, B: np.ndarray, fmt: str = "binary64") -> Tuple[np.ndarray, np.ndarray]:
    """The enclosure of A @ B: exact product, rounded outward once."""
    S, Q = product_exact_scaled(A, B)
    return enclose_from_integer(S, Q, fmt)


def enclose_brute_force(A: np.ndarray, B: np.ndarray, fmt: str = "binary64") -> Tuple[np.ndarray, np.ndarray]:
    """The same pair from the term-by-term Fraction sum (tiny inputs)."""
    V = product_exact_fractions(A, B)
    dt = np.float64 if fmt == "binary64" else np.float32
    lo = np.empty(V.shape, dtype=dt)
    hi = np.empty(V.shape, dtype=dt)
    for idx, v in np.ndenumerate(V):
        lo[idx] = round_down(v, fmt)
        hi[idx] = round_up(v, fmt)
    return lo, hi
