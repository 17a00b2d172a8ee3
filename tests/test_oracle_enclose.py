"""Pins of the enclosure oracle (oracle/enclose.py) against the mathematics
and library routines, independent of the oracle's own formulas."""
import math
import sys
from fractions import Fraction

import numpy as np
import pytest

from oracle import enclose as E

DBL_MAX = sys.float_info.max
DBL_TRUE_MIN = math.ldexp(1.0, -1074)
FLT_MAX = float(np.finfo(np.float32).max)


def _random_doubles(rng, n):
    """Finite doubles over the whole exponent range, subnormals and signs included."""
    bits = rng.integers(0, 2 ** 63, size=n, dtype=np.uint64) | (rng.integers(0, 2, size=n, dtype=np.uint64) << np.uint64(63))
    x = bits.view(np.float64)
    return [float(v) for v in x if math.isfinite(v)]


def test_representable_values_are_fixed_points():
    rng = np.random.default_rng(1)
    xs = _random_doubles(rng, 400) + [0.0, DBL_MAX, -DBL_MAX, DBL_TRUE_MIN, -DBL_TRUE_MIN,
                                      math.ldexp(1.0, -1022), 1.0, -3.5]
    for x in xs:
        v = E.exact(x)
        assert E.round_down(v) == x and E.round_up(v) == x


def test_directed_rounding_matches_nextafter():
    """Just above / below a double: the neighbours are math.nextafter's."""
    rng = np.random.default_rng(2)
    for x in _random_doubles(rng, 300) + [DBL_TRUE_MIN, -DBL_TRUE_MIN, math.ldexp(1.0, -1022)]:
        if abs(x) == DBL_MAX:
            continue
        up = math.nextafter(x, math.inf)
        down = math.nextafter(x, -math.inf)
        eps_up = (E.exact(up) - E.exact(x)) / 3
        eps_dn = (E.exact(x) - E.exact(down)) / 3
        assert E.round_down(E.exact(x) + eps_up) == x
        assert E.round_up(E.exact(x) + eps_up) == up
        assert E.round_up(E.exact(x) - eps_dn) == x
        assert E.round_down(E.exact(x) - eps_dn) == down


def test_binary32_matches_numpy_nextafter():
    rng = np.random.default_rng(3)
    xs = rng.standard_normal(200).astype(np.float32) * np.float32(2.0) ** rng.integers(-140, 120, 200).astype(np.float32)
    for x in xs:
        x = np.float32(x)
        if not np.isfinite(x) or x == 0:
            continue
        up = np.nextafter(x, np.float32(np.inf))
        v = E.exact(float(x)) + (E.exact(float(up)) - E.exact(float(x))) / 5
        assert E.round_down(v, "binary32") == float(x)
        assert E.round_up(v, "binary32") == float(up)


def test_overflow_saturates_inward_and_goes_to_infinity_outward():
    big = Fraction(2) ** 1024
    assert (E.round_down(big), E.round_up(big)) == (DBL_MAX, math.inf)
    assert (E.round_down(-big), E.round_up(-big)) == (-math.inf, -DBL_MAX)
    just = E.exact(DBL_MAX) + Fraction(1, 10 ** 9)
    assert (E.round_down(just), E.round_up(just)) == (DBL_MAX, math.inf)
    b32 = Fraction(2) ** 128
    assert (E.round_down(b32, "binary32"), E.round_up(b32, "binary32")) == (FLT_MAX, math.inf)


def test_subnormal_boundary():
    half_min = Fraction(1, 2 ** 1075)
    assert (E.round_down(half_min), E.round_up(half_min)) == (0.0, DBL_TRUE_MIN)
    assert (E.round_down(-half_min), E.round_up(-half_min)) == (-DBL_TRUE_MIN, 0.0)
    largest_sub = math.ldexp(1.0, -1022) - DBL_TRUE_MIN
    mid = (E.exact(largest_sub) + E.exact(math.ldexp(1.0, -1022))) / 2
    assert (E.round_down(mid), E.round_up(mid)) == (largest_sub, math.ldexp(1.0, -1022))


def test_lowest_set_bit_and_scale():
    assert E.lowest_set_bit_exponent(1.0) == 0
    assert E.lowest_set_bit_exponent(12.0) == 2
    assert E.lowest_set_bit_exponent(0.375) == -3
    assert E.lowest_set_bit_exponent(DBL_TRUE_MIN) == -1074
    X = np.array([[0.5, 3.0], [0.0, -0.125]])
    F = E.coarsest_lossless_scale(X)
    assert F == 3
    S = E.scaled_integers(X, F)
    assert S.tolist() == [[4, 24], [0, -1]]
    assert E.coarsest_lossless_scale(np.zeros((2, 2))) == 0
    with pytest.raises(ValueError):
        E.coarsest_lossless_scale(np.array([1.0, np.inf]))


def test_integer_operands_equal_int64_product():
    """Integer operands: the product is an integer and (if representable)
    lo == hi == the int64 product (enclosure-gemm, "Correctness")."""
    rng = np.random.default_rng(4)
    A = rng.integers(-1000, 1000, size=(7, 11))
    B = rng.integers(-1000, 1000, size=(11, 5))
    lo, hi = E.enclose(A.astype(np.float64), B.astype(np.float64))
    ref = (A @ B).astype(np.float64)
    assert np.array_equal(lo, ref) and np.array_equal(hi, ref)


def test_catastrophic_cancellation():
    A = np.array([[1e16, 1.0, -1e16, 2.0 ** -60]])
    B = np.array([[1.0], [1.0], [1.0], [1.0]])
    lo, hi = E.enclose(A, B)
    v = 1 + Fraction(1, 2 ** 60)
    assert lo[0, 0] == 1.0 and hi[0, 0] == math.nextafter(1.0, 2.0)
    assert E.exact(lo[0, 0]) <= v <= E.exact(hi[0, 0])


@pytest.mark.parametrize("seed", [5, 6, 7])
def test_scaled_product_equals_brute_force(seed):
    rng = np.random.default_rng(seed)
    A = rng.standard_normal((4, 6)) * 2.0 ** rng.integers(-30, 30, size=(4, 6))
    B = rng.standard_normal((6, 3)) * 2.0 ** rng.integers(-30, 30, size=(6, 3))
    A[1, 2] = 0.0
    A[2, 3] = math.ldexp(1.0, -1060)        # subnormal
    S, Q = E.product_exact_scaled(A, B)
    V = E.product_exact_fractions(A, B)
    for idx, s in np.ndenumerate(S):
        assert Fraction(int(s), 2 ** Q) == V[idx]
    lo, hi = E.enclose(A, B)
    blo, bhi = E.enclose_brute_force(A, B)
    assert np.array_equal(lo, blo) and np.array_equal(hi, bhi)


def test_bracket_is_one_step_and_contains():
    rng = np.random.default_rng(8)
    A = rng.standard_normal((5, 40))
    B = rng.standard_normal((40, 4))
    lo, hi = E.enclose(A, B)
    V = E.product_exact_fractions(A, B)
    for idx, v in np.ndenumerate(V):
        assert E.exact(lo[idx]) <= v <= E.exact(hi[idx])
        assert hi[idx] == lo[idx] or hi[idx] == math.nextafter(lo[idx], math.inf)


def test_enclosure_digest_inputs():
    """The stored enclosure digest was made from the inputs the generator draws."""
    import hashlib
    import json
    import os
    import workloads as W
    dg = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "enclosure_digest.json")))
    A, B = W.fp64_normal_pair(dg["seed"], dg["M"], dg["K"], dg["N"])
    assert hashlib.sha256(A.tobytes()).hexdigest() == dg["inputs_sha256"]["A"]
    assert hashlib.sha256(B.tobytes()).hexdigest() == dg["inputs_sha256"]["B"]
    assert (E.coarsest_lossless_scale(A), E.coarsest_lossless_scale(B)) == (dg["Fa"], dg["Fb"])
