"""Plain definitions for the exact rational solve A x = b by Dixon p-adic
lifting (page "exact-solve").

TEST INFRASTRUCTURE ONLY: imported by the test suite, the smoke check and the
``cpu_baseline`` leg of ``bench.py``; never by the product path.

Follows exact-solve:

* "Method": with B = A^-1 mod P, r_0 = b, x_i = B r_i mod P and
  r_{i+1} = (r_i - A x_i) / P, the digits x_i give x mod P^m; the solution is
  recovered once P^m exceeds twice the Hadamard bound on numerator and
  denominator.  P is a product of primes below 256; A^-1 mod each prime comes
  from Gauss-Jordan elimination of the augmented matrix [A | I].
* "Correctness": the reference is an exact Fraction Gaussian elimination; at
  larger sizes the identity A @ N == d * b (numerators N, common denominator
  d) is checked.
* "Requirements and limits": n * max|A_ij| < 2^63 keeps the residual in one
  signed 64-bit limb.

Readings taken where the page is silent:
  * the lift's primes are the odd primes below 256 for which A is invertible;
    P must be odd (the residual update divides by P modulo 2^64);
  * the digit x_i is the balanced representative of B r_i mod P;
  * the step count m is the least with P^m > 2 * N_bound * D_bound, where
    D_bound is Hadamard's bound on |det A| (product of row norms) and N_bound
    the same with b's column in place of A's weakest column (a bound on every
    Cramer numerator);
  * the rational value of each component is the unique N/d with |N| <=
    N_bound, 0 < d <= D_bound and N = d * (x mod P^m) (mod P^m), found by the
    extended Euclidean algorithm.

Pins: tests/test_oracle_dixon.py (Fraction solve against A x == b and a
planted integer solution; modular inverses against A B = I mod q; the lift
against A X = b mod P^m; rational reconstruction of known fractions).
"""
from __future__ import annotations

import math
from fractions import Fraction
from typing import List, Optional, Sequence, Tuple

import numpy as np

from . import oracle as O


def solve_fraction(A: Sequence[Sequence[int]], b: Sequence[Sequence[int]]) -> Optional[List[List[Fraction]]]:
    """Gaussian elimination in exact rationals; None when A is singular."""
    n = len(A)
    c = len(b[0])
    M = [[Fraction(int(A[i][j])) for j in range(n)] + [Fraction(int(b[i][k])) for k in range(c)]
         for i in range(n)]
    for k in range(n):
        p = next((i for i in range(k, n) if M[i][k] != 0), None)
        if p is None:
            return None
        M[k], M[p] = M[p], M[k]
        piv = M[k][k]
        M[k] = [v / piv for v in M[k]]
        for i in range(n):
            if i != k and M[i][k] != 0:
                f = M[i][k]
                M[i] = [vi - f * vk for vi, vk in zip(M[i], M[k])]
    return [[M[i][n + k] for k in range(c)] for i in range(n)]


def inverse_mod(A: Sequence[Sequence[int]], q: int) -> Optional[List[List[int]]]:
    """A^-1 mod q (entries in [0, q)) by Gauss-Jordan on [A | I]; None if
    A is singular mod q."""
    n = len(A)
    M = [[int(A[i][j]) % q for j in range(n)] + [1 if j == i else 0 for j in range(n)] for i in range(n)]
    for k in range(n):
        p = next((i for i in range(k, n) if M[i][k] != 0), None)
        if p is None:
            return None
        M[k], M[p] = M[p], M[k]
        inv = pow(M[k][k], -1, q)
        M[k] = [v * inv % q for v in M[k]]
        for i in range(n):
            if i != k and M[i][k] != 0:
                f = M[i][k]
                M[i] = [(vi - f * vk) % q for vi, vk in zip(M[i], M[k])]
    return [row[n:] for row in M]


def lift_primes(A: Sequence[Sequence[int]], candidates: Optional[Sequence[int]] = None) -> List[int]:
    """The odd primes below 256 (largest first) for which A is invertible."""
    cands = [q for q in O.primes_largest_first() if q % 2] if candidates is None else list(candidates)
    return [q for q in cands if inverse_mod(A, q) is not None]


def hadamard_bounds(A: Sequence[Sequence[int]], b: Sequence[Sequence[int]]) -> Tuple[int, int]:
    """(N_bound, D_bound): |det A| <= D_bound, |every Cramer numerator| <= N_bound.

    D = prod of the row norms of A (Hadamard); a numerator is the determinant
    of A with one column replaced by a column of b, so its rows are A's rows
    with one entry changed: each row norm is at most sqrt(||a_i||^2 + b_i^2),
    over the worst column of b.  Integer ceilings of the square roots keep the
    bounds rigorous."""
    n = len(A)
    c = len(b[0])
    rows2 = [sum(int(v) ** 2 for v in A[i]) for i in range(n)]
    D = 1
    for r2 in rows2:
        D *= math.isqrt(r2) + (0 if math.isqrt(r2) ** 2 == r2 else 1)
    N = 0
    for k in range(c):
        Nk = 1
        for i in range(n):
            r2 = rows2[i] + int(b[i][k]) ** 2
            Nk *= math.isqrt(r2) + (0 if math.isqrt(r2) ** 2 == r2 else 1)
        N = max(N, Nk)
    return max(N, 1), max(D, 1)


def lift_steps(P: int, N_bound: int, D_bound: int) -> int:
    """The least m with P^m > 2 * N_bound * D_bound."""
    m, Pm = 1, P
    while Pm <= 2 * N_bound * D_bound:
        m += 1
        Pm *= P
    return m


def dixon_digits(A: Sequence[Sequence[int]], b: Sequence[Sequence[int]], primes: Sequence[int],
                 steps: int) -> List[List[List[int]]]:
    """The page's recurrence in Python integers: x_i = B r_i mod P (balanced),
    r_{i+1} = (r_i - A x_i) / P, with B = A^-1 mod P assembled by CRT from the
    per-prime inverses.  Returns digits[i][row][col]."""
    n = len(A)
    c = len(b[0])
    P = O.prod(primes)
    invs = [inverse_mod(A, q) for q in primes]
    Bm = [[O.crt_balanced([invs[t][i][j] for t in range(len(primes))], primes) % P for j in range(n)]
          for i in range(n)]
    r = [[int(b[i][k]) for k in range(c)] for i in range(n)]
    digits = []
    for _ in range(steps):
        x = [[O.balanced(sum(Bm[i][j] * r[j][k] for j in range(n)), P) for k in range(c)] for i in range(n)]
        digits.append(x)
        Ax = [[sum(int(A[i][j]) * x[j][k] for j in range(n)) for k in range(c)] for i in range(n)]
        nxt = []
        for i in range(n):
            row = []
            for k in range(c):
                t = r[i][k] - Ax[i][k]
                assert t % P == 0
                row.append(t // P)
            nxt.append(row)
        r = nxt
    return digits


def padic_value(digits: Sequence[Sequence[Sequence[int]]], P: int) -> List[List[int]]:
    """X = sum_i digits[i] * P^i, componentwise."""
    n = len(digits[0])
    c = len(digits[0][0])
    X = [[0] * c for _ in range(n)]
    Pi = 1
    for d in digits:
        for i in range(n):
            for k in range(c):
                X[i][k] += d[i][k] * Pi
        Pi *= P
    return X


def rational_reconstruct(u: int, M: int, N_bound: int, D_bound: int) -> Optional[Fraction]:
    """The N/d with |N| <= N_bound, 0 < d <= D_bound and N = d u (mod M), by
    the extended Euclidean algorithm on (M, u mod M); unique when
    M > 2 N_bound D_bound.  None if there is none."""
    r0, r1 = M, u % M
    t0, t1 = 0, 1
    while r1 > N_bound:
        qt = r0 // r1
        r0, r1 = r1, r0 - qt * r1
        t0, t1 = t1, t0 - qt * t1
    if t1 == 0 or abs(t1) > D_bound:
        return None
    if (r1 - t1 * u) % M != 0:
        return None
    return Fraction(r1, t1)


def solve_dixon(A, b, primes: Optional[Sequence[int]] = None) -> Optional[List[List[Fraction]]]:
    """The whole method in Python integers (small systems)."""
    ps = lift_primes(A) if primes is None else list(primes)
    if not ps:
        return None
    P = O.prod(ps)
    Nb, Db = hadamard_bounds(A, b)
    m = lift_steps(P, Nb, Db)
    X = padic_value(dixon_digits(A, b, ps, m), P)
    M = P ** m
    out = []
    for row in X:
        vals = []
        for u in row:
            f = rational_reconstruct(u, M, Nb, Db)
            if f is None:
                return None
            vals.append(f)
        out.append(vals)
    return out
