"""Pins of the Dixon-lift oracle (oracle/dixon.py) against exact identities
and independent routines (sympy determinants, Python's modular inverse)."""
import math
import random
from fractions import Fraction

import numpy as np
import pytest

from oracle import dixon as D
from oracle import oracle as O


def _system(seed, n, c, amax=1000, bmax=1000):
    rng = random.Random(seed)
    A = [[rng.randint(-amax, amax) for _ in range(n)] for _ in range(n)]
    b = [[rng.randint(-bmax, bmax) for _ in range(c)] for _ in range(n)]
    return A, b


def _matmul(A, X):
    return [[sum(A[i][k] * X[k][j] for k in range(len(X))) for j in range(len(X[0]))] for i in range(len(A))]


@pytest.mark.parametrize("seed,n,c", [(1, 5, 1), (2, 8, 3), (3, 12, 2)])
def test_fraction_solve_satisfies_the_system(seed, n, c):
    A, b = _system(seed, n, c)
    X = D.solve_fraction(A, b)
    assert _matmul(A, X) == [[Fraction(v) for v in row] for row in b]


def test_fraction_solve_planted_and_singular():
    A, _ = _system(4, 7, 1)
    x = [[3], [-1], [0], [7], [2], [-5], [11]]
    b = _matmul(A, x)
    assert D.solve_fraction(A, b) == [[Fraction(v[0])] for v in x]
    S = [row[:] for row in A]
    S[6] = [S[0][j] + 2 * S[1][j] for j in range(7)]        # dependent row
    assert D.solve_fraction(S, b) is None


@pytest.mark.parametrize("q", [3, 5, 251, 127])
def test_inverse_mod_is_an_inverse(q):
    A, _ = _system(5, 9, 1)
    B = D.inverse_mod(A, q)
    if B is None:
        pytest.skip("singular mod q for this seed")
    AB = _matmul(A, B)
    assert all((AB[i][j] - (1 if i == j else 0)) % q == 0 for i in range(9) for j in range(9))


def test_inverse_mod_singular():
    A = [[1, 2, 3], [4, 5, 6], [7, 8, 10]]                # det = -3
    assert D.inverse_mod(A, 3) is None
    assert D.inverse_mod(A, 5) is not None
    assert 3 not in D.lift_primes(A) and 5 in D.lift_primes(A)


def test_hadamard_bounds_hold():
    import sympy
    for seed in range(6, 10):
        A, b = _system(seed, 6, 2, 50, 50)
        Nb, Db = D.hadamard_bounds(A, b)
        detA = int(sympy.Matrix(A).det())
        assert abs(detA) <= Db
        for k in range(2):
            for j in range(6):
                Aj = [row[:] for row in A]
                for i in range(6):
                    Aj[i][j] = b[i][k]
                assert abs(int(sympy.Matrix(Aj).det())) <= Nb


def test_rational_reconstruction_of_known_fractions():
    rng = random.Random(11)
    M = O.prod(O.primes_largest_first()[:8])
    Nb = Db = math.isqrt(M // 2) - 1
    for _ in range(200):
        d = rng.randint(1, Db)
        while math.gcd(d, M) != 1:            # denominators are coprime to P (det A is)
            d = rng.randint(1, Db)
        n = rng.randint(-Nb, Nb)
        u = n * pow(d, -1, M) % M
        assert D.rational_reconstruct(u, M, Nb, Db) == Fraction(n, d)


@pytest.mark.parametrize("seed,n,c", [(12, 6, 1), (13, 9, 2), (14, 5, 3)])
def test_lift_digits_solve_the_system_mod_P_power(seed, n, c):
    A, b = _system(seed, n, c)
    ps = D.lift_primes(A)[:6]
    P = O.prod(ps)
    digits = D.dixon_digits(A, b, ps, 4)
    X = D.padic_value(digits, P)
    AX = _matmul(A, X)
    M = P ** 4
    assert all((AX[i][k] - b[i][k]) % M == 0 for i in range(n) for k in range(c))
    for d in digits:
        assert all(2 * abs(v) < P for row in d for v in row)


@pytest.mark.parametrize("seed,n,c", [(15, 6, 1), (16, 10, 2), (17, 4, 4)])
def test_dixon_equals_fraction_solve(seed, n, c):
    A, b = _system(seed, n, c)
    assert D.solve_dixon(A, b) == D.solve_fraction(A, b)


def test_dixon_scaled_hilbert():
    """A scaled Hilbert system: dense denominators (exact-solve, "Correctness")."""
    n = 6
    L = math.lcm(*range(1, 2 * n))
    A = [[L // (i + j + 1) for j in range(n)] for i in range(n)]
    b = [[1] for _ in range(n)]
    X = D.solve_dixon(A, b)
    assert X == D.solve_fraction(A, b)
    assert max(x[0].denominator for x in X) > 1
