"""The host stage of the exact solve (bounds, step count, rational
reconstruction of the lift digits) against the oracle, on the CPU: the digits
come from the oracle's own recurrence."""
import random

import numpy as np
import pytest

from exact_integer_gemm_amd import exact_solve as S
from oracle import dixon as D
from oracle import oracle as O


def _system(seed, n, c, amax=1000, bmax=1000):
    rng = random.Random(seed)
    A = [[rng.randint(-amax, amax) for _ in range(n)] for _ in range(n)]
    b = [[rng.randint(-bmax, bmax) for _ in range(c)] for _ in range(n)]
    return A, b


@pytest.mark.parametrize("seed,n,c", [(1, 6, 1), (2, 9, 3), (3, 4, 2)])
def test_reconstruction_from_oracle_digits(seed, n, c):
    A, b = _system(seed, n, c)
    ps = D.lift_primes(A)
    P = O.prod(ps)
    Nb, Db = S._bounds(np.array(A, dtype=np.int64), np.array(b, dtype=np.int64))
    assert (Nb, Db) == D.hadamard_bounds(A, b)
    m = S.lift_steps_for(P, Nb, Db)
    assert P ** m > 2 * Nb * Db * (Db + 1) and P ** (m - 1) <= 2 * Nb * Db * (Db + 1)
    digits = D.dixon_digits(A, b, ps, m)
    per_step = [[digits[s][i][k] for i in range(n) for k in range(c)] for s in range(m)]
    nums, den = S.reconstruct(per_step, P, m, Nb, Db)
    ref = D.solve_fraction(A, b)
    assert [[S.Fraction(nums[i * c + k], den) for k in range(c)] for i in range(n)] == ref


def test_limbs_to_int_matches_the_oracle():
    rng = np.random.default_rng(4)
    L = rng.integers(-2 ** 63, 2 ** 63 - 1, size=(7, 5, 3), dtype=np.int64)
    assert S._limbs_to_int(L) == [int(v) for v in O.decode_array(L).ravel()]


def test_odd_primes():
    assert S.ODD_PRIMES == [q for q in O.primes_largest_first() if q % 2]
