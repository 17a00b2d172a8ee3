"""The host stage of the exact solve (bounds, step count, rational
reconstruction of the lift digits) against the oracle, on the CPU: the digits
come from the oracle's own recurrence."""
import math
from fractions import Fraction
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


# ---- the native host stage (GMP through the library; host pointers only) -------------------

def _native():
    import exact_integer_gemm_amd as rg
    try:
        rg.load()
    except Exception as e:          # the library is missing: nothing native to test
        pytest.skip(f"library not built: {e}")
    if not S.host_bigint_available():
        pytest.skip("libgmp.so.10 is not available")


def _digit_array(digits_per_step, L):
    """Python-int digits [m][count] -> int64 [m][count][L] two's-complement limbs."""
    m, cnt = len(digits_per_step), len(digits_per_step[0])
    out = np.zeros((m, cnt, L), dtype=np.int64)
    for s in range(m):
        for i in range(cnt):
            out[s, i] = O.to_limbs(int(digits_per_step[s][i]), L)
    return out


@pytest.mark.parametrize("seed,n,c", [(1, 6, 1), (2, 9, 3), (5, 12, 2)])
def test_native_reconstruction_from_oracle_digits(seed, n, c):
    _native()
    A, b = _system(seed, n, c)
    ps = D.lift_primes(A)
    P = O.prod(ps)
    Nb, Db = D.hadamard_bounds(A, b)
    m = S.lift_steps_for(P, Nb, Db)
    digits = D.dixon_digits(A, b, ps, m)
    per_step = [[digits[s][i][k] for i in range(n) for k in range(c)] for s in range(m)]
    L = (P.bit_length() + 64) // 64
    nums, den = S.reconstruct_digits(_digit_array(per_step, L), P, m, Nb, Db)
    ref = D.solve_fraction(A, b)
    assert [[S.Fraction(nums[i * c + k], den) for k in range(c)] for i in range(n)] == ref


def test_native_padic_value_matches_the_oracle():
    """D = 1 and the widest bound give X = sum_s digits[s] P^s itself."""
    _native()
    rng = random.Random(6)
    for ps, m, cnt in ((O.primes_largest_first()[1:9], 7, 11), ([3], 1, 4), ([251, 241, 239], 33, 5)):
        P = O.prod(ps)
        per_step = [[rng.randint(-(P // 2), P // 2) for _ in range(cnt)] for _ in range(m)]
        L = (P.bit_length() + 64) // 64
        ok, X = S.padic_numerators(_digit_array(per_step, L), P, 1, P ** m // 2)
        ref = D.padic_value([[[v] for v in row] for row in per_step], P)
        assert ok.all() and X == [r[0] for r in ref]


def test_native_common_denominator_test():
    """Planted fractions a/e: with D a multiple of every e the numerator D a / e is accepted; with
    D = 1 only the integer components are (the rest exceed the bound), never a wrong value."""
    _native()
    rng = random.Random(7)
    ps = [q for q in O.primes_largest_first() if q % 2][:10]
    P = O.prod(ps)
    m = 9
    Pm = P ** m
    Nb = 2 ** 60
    es = [2 ** 50 + 1, 1, 3 ** 20, 2 ** 40 + 3, 1]
    assert all(math.gcd(e, P) == 1 for e in es)
    comps = [(rng.randint(-Nb, Nb), e) for e in es]
    vals = [a * pow(e, -1, Pm) % Pm for a, e in comps]
    vals = [u - Pm if u > Pm // 2 else u for u in vals]
    per_step = []
    for _ in range(m):
        row = []
        for i, v in enumerate(vals):
            d = O.balanced(v, P)
            vals[i] = (v - d) // P
            row.append(d)
        per_step.append(row)
    dig = _digit_array(per_step, (P.bit_length() + 64) // 64)
    Dfull = math.lcm(*es)
    assert Pm > 2 * Dfull * Nb * (Dfull + 1)
    ok, w = S.padic_numerators(dig, P, Dfull, Dfull * Nb)
    assert ok.all() and w == [a * (Dfull // e) for a, e in comps]
    ok1, w1 = S.padic_numerators(dig, P, 1, Nb)
    assert list(ok1) == [e == 1 for _, e in comps]
    assert [w1[i] for i in range(len(es)) if ok1[i]] == [a for a, e in comps if e == 1]
    ok_t, w_t = S.padic_numerators(dig, P, Dfull, Dfull * Nb, threads=1)
    assert list(ok_t) == list(ok) and w_t == w
    nums, den = S.reconstruct_digits(dig, P, m, Nb, Dfull)
    assert [S.Fraction(v, den) for v in nums] == [S.Fraction(a, e) for a, e in comps]
    assert den == math.lcm(*[S.Fraction(a, e).denominator for a, e in comps])   # lowest terms


def test_native_rational_reconstruction_matches_the_oracle():
    _native()
    rng = random.Random(8)
    M = O.prod(O.primes_largest_first()[1:12])
    Nb = Db = math.isqrt(M // 2) - 1
    for _ in range(150):
        d = rng.randint(1, Db)
        while math.gcd(d, M) != 1:
            d = rng.randint(1, Db)
        a = rng.randint(-Nb, Nb)
        u = a * pow(d, -1, M) % M
        assert S.rational_reconstruct(u, M, Nb, Db) == D.rational_reconstruct(u, M, Nb, Db) == S.Fraction(a, d)
    # tight bounds: residues with no small fraction; both sides agree on None or the value
    for _ in range(150):
        u = rng.randrange(M)
        assert S.rational_reconstruct(u, M, 2 ** 20, 2 ** 20) == D.rational_reconstruct(u, M, 2 ** 20, 2 ** 20)


def test_native_host_stage_argument_errors():
    _native()
    import ctypes
    import exact_integer_gemm_amd as rg
    lib = rg.load()
    dig = np.zeros((2, 3, 1), dtype=np.int64)
    one = np.ones(1, dtype=np.uint64)
    P = np.array([15], dtype=np.uint64)
    Peven = np.array([16], dtype=np.uint64)
    big = np.array([0, 1], dtype=np.uint64)          # 2^64
    num = np.zeros((3, 1), dtype=np.int64)
    ok = np.zeros(3, dtype=np.int32)
    p = lambda a: a.ctypes.data

    def call(idx, Pv=P, bound=one, bl=1, wl=1):
        ix = np.array(idx, dtype=np.int64)
        return lib.rns_padic_numerators(p(dig), 2, 3, 1, p(ix), len(ix), p(Pv), 1, p(one), 1, p(bound), bl,
                                        p(num), wl, p(ok), 1)
    assert call([0, 1, 2]) == 0
    assert call([3]) == -1                             # index beyond count
    assert call([-1]) == -1
    assert call([0], Pv=Peven) == -1                   # P must be odd
    assert call([0], bound=big, bl=2) == -4            # bound does not fit one signed limb
    assert call([0], bound=big, bl=2, wl=2) == 0
    assert lib.rns_error_string(-8).decode() and lib.rns_error_string(-9).decode()
    d = np.zeros(1, dtype=np.uint64)
    assert lib.rns_rational_reconstruct(p(one), 1, p(np.zeros(1, dtype=np.uint64)), 1, p(one), 1, p(one), 1,
                                        p(num), 1, p(d), 1) == -1  # M = 0


def test_native_rational_reconstruction_long_remainder_sequences():
    """Moduli of thousands of bits with bounds far below them, so that the reconstruction runs
    through its batched (Lehmer) steps before the last single divisions: the fraction equals the
    oracle's, for planted fractions and for residues with no fraction within the bounds."""
    _native()
    rng = random.Random(9)
    ps = [q for q in O.primes_largest_first() if q % 2]
    for bits, nb_bits, trials in ((4000, 1500, 12), (20000, 9000, 3), (600, 100, 30)):
        M = 1
        while M.bit_length() < bits:
            M *= ps[rng.randrange(len(ps))]
        Nb = rng.getrandbits(nb_bits) | (1 << (nb_bits - 1))
        Db = (M // (2 * Nb)) - 1
        for _ in range(trials):
            d = rng.randint(1, Db)
            while math.gcd(d, M) != 1:
                d = rng.randint(1, Db)
            a = rng.randint(-Nb, Nb)
            u = a * pow(d, -1, M) % M
            assert S.rational_reconstruct(u, M, Nb, Db) == D.rational_reconstruct(u, M, Nb, Db) == S.Fraction(a, d)
            v = rng.randrange(M)
            small = 2 ** (nb_bits // 2)
            assert S.rational_reconstruct(v, M, small, small) == D.rational_reconstruct(v, M, small, small)


def test_pow_table_chunks():
    P = O.prod([251, 241, 239, 233])
    tab = S.pow_table(P, 5, 6)
    for s in range(5):
        v = sum(int(tab[t, s]) << (32 * t) for t in range(6))
        assert v == P ** s and all(0 <= int(x) < 2 ** 32 for x in tab[:, s])


def test_pow_table_wide_and_too_narrow():
    """All 54 primes (P near 2^335): 11 powers over 116 chunks; too few chunks is an error."""
    P = O.prod(O.primes_largest_first())
    tab = S.pow_table(P, 11, 116)
    for s in range(11):
        assert sum(int(tab[t, s]) << (32 * t) for t in range(116)) == P ** s
    if S.host_bigint_available():
        with pytest.raises(Exception):
            S.pow_table(P, 11, 100)


def test_native_numerators_from_chunks_equal_from_digits():
    """The same numerators whether the p-adic values come as digits or as binary chunks."""
    _native()
    rng = random.Random(10)
    ps = [q for q in O.primes_largest_first() if q % 2][:12]
    P = O.prod(ps)
    m, cnt = 9, 13
    per_step = [[rng.randint(-(P // 2), P // 2) for _ in range(cnt)] for _ in range(m)]
    L = (P.bit_length() + 64) // 64
    dig = _digit_array(per_step, L)
    X = [r[0] for r in D.padic_value([[[v] for v in row] for row in per_step], P)]
    T = ((P ** m).bit_length() + 1 + 31) // 32
    chunks = np.array([[(x % (1 << (32 * T))) >> (32 * t) & 0xffffffff for t in range(T)] for x in X],
                      dtype=np.uint32)
    Dd = 3 * 7 * 2 ** 40 + 1
    for Dv, bound in ((1, P ** m // 2), (Dd, Dd * 2 ** 200)):
        ok1, w1 = S.padic_numerators(dig, P, Dv, bound)
        ok2, w2 = S.chunk_numerators(chunks, P, m, Dv, bound)
        assert list(ok1) == list(ok2) and w1 == w2
    ok, w = S.chunk_numerators(chunks, P, m, 1, P ** m // 2)
    assert ok.all() and w == X


def _barrett_step(X, D, c, Pm):
    """The integer function rns_chunk_modmul computes, in Python integers."""
    Y = D * X
    a = Y >> (32 * c.s1c)
    mu = sum(int(v) << (32 * i) for i, v in enumerate(c.mu.tolist()))
    q = (a * mu + (1 << (32 * c.k2c - 1))) >> (32 * c.k2c)
    return Y - q * Pm


@pytest.mark.parametrize("n_primes,m,dbits", [(3, 5, 40), (12, 40, 900), (50, 30, 3000)])
def test_modmul_constants_leave_one_correction(n_primes, m, dbits):
    """The Barrett constants: for every D <= Db and |X| <= P^m / 2, D X - q P^m is congruent to
    D X mod P^m and below P^m in magnitude (one +-P^m correction gives the balanced residue), and
    fits the Tw output chunks; extremes of D and X included."""
    P = O.prod(O.primes_largest_first()[1:1 + n_primes])
    Pm = P ** m
    Db = (1 << dbits) - 1
    c = S.ModmulConstants(P, m, Db, "cpu")
    assert sum(int(v) << (32 * i) for i, v in enumerate(c.Pm.tolist())) == Pm
    rng = random.Random(n_primes)
    half = (Pm - 1) // 2
    cases = [(Db, half), (Db, -half), (1, half), (Db, 0), (Db - 1, -1)]
    cases += [(rng.randrange(1, Db + 1), rng.randrange(-half, half + 1)) for _ in range(200)]
    for D, X in cases:
        w0 = _barrett_step(X, D, c, Pm)
        assert (w0 - D * X) % Pm == 0
        assert abs(w0) < Pm and abs(w0) < 2 ** (32 * c.Tw - 1)
        assert abs(w0) <= Pm // 2 + Pm // 2 ** 60


def _lane_sub_mod(wv, fc, q):
    """Four bytes a - c mod q (a, c in [0, q)) two at a time in 16-bit lanes, as the panel
    elimination forms them: 256 + a - c per lane, then + q where bit 8 is clear."""
    M = 0xFFFFFFFF
    qq = q | (q << 16)
    x = (((wv & 0x00FF00FF) | 0x01000100) - (fc & 0x00FF00FF)) & M
    y = ((((wv >> 8) & 0x00FF00FF) | 0x01000100) - ((fc >> 8) & 0x00FF00FF)) & M
    mx, my = ((~x & M) >> 8) & 0x00010001, ((~y & M) >> 8) & 0x00010001
    x = (x + ((((mx << 8) - mx) & M) & qq)) & 0x00FF00FF
    y = (y + ((((my << 8) - my) & M) & qq)) & 0x00FF00FF
    return (x | (y << 8)) & M


def test_panel_lane_subtraction_every_prime():
    """The byte arithmetic of the panel elimination equals (a - c) mod q bytewise for every odd
    prime below 256, at the extremes 0 and q - 1 and on random bytes."""
    rng = random.Random(3)
    for q in [p for p in O.primes_largest_first() if p % 2]:
        cases = [[rng.choice([0, q - 1]) for _ in range(8)] for _ in range(200)]
        cases += [[rng.randrange(q) for _ in range(8)] for _ in range(500)]
        for v in cases:
            a, c = v[:4], v[4:]
            wv = sum(x << (8 * b) for b, x in enumerate(a))
            fc = sum(x << (8 * b) for b, x in enumerate(c))
            assert _lane_sub_mod(wv, fc, q) == sum(((a[b] - c[b]) % q) << (8 * b) for b in range(4)), q


def test_pow2_quotient_native():
    """floor(2^e / d) from GMP equals Python's integer division (the Barrett reciprocal)."""
    _native()
    rng = random.Random(4)
    for _ in range(40):
        d = rng.getrandbits(rng.randrange(1, 3000)) | 1
        e = rng.randrange(0, 6000)
        ql = max(1, (e - d.bit_length() + 1) // 64 + 2)
        q = np.zeros(ql, dtype=np.uint64)
        dl, dn = S._mag(d)
        assert S.load().rns_pow2_quotient(e, S._ptr(dl), dn, S._ptr(q), ql) == 0
        assert int.from_bytes(q.tobytes(), "little") == (1 << e) // d


def test_step_count_and_sample_modulus_are_least():
    """The lift's step count is the least m with P^m > 2 Nb Db (Db + 1), and the sample's modulus
    the least power P^k > 2 Nb Db, across sizes (computed from bit lengths, then corrected)."""
    rng = random.Random(5)
    odd = [p for p in O.primes_largest_first() if p % 2]
    for _ in range(300):
        P = O.prod(rng.sample(odd, rng.randrange(1, 8)))
        Nb, Db = rng.getrandbits(rng.randrange(1, 900)) + 1, rng.getrandbits(rng.randrange(1, 900)) + 1
        m = S.lift_steps_for(P, Nb, Db)
        target = 2 * Nb * Db * (Db + 1)
        assert P ** m > target and (m == 1 or P ** (m - 1) <= target)
        Pk = S._sample_modulus(P, Nb, Db)
        assert Pk > 2 * Nb * Db and (Pk == P or Pk // P <= 2 * Nb * Db)
        assert Pk % P == 0 and round(math.log(Pk, P)) >= 1


def test_fractions_in_lowest_terms_native():
    """Batched reduction N_i / D: equal to Fraction's own normalisation, signs, zero and shared
    factors included."""
    _native()
    rng = random.Random(6)
    D = 2 ** 5 * 3 ** 7 * 251 * (rng.getrandbits(3000) | 1)
    nums = [0, 1, -1, D, -D, 2 * D, 3 ** 5, -(2 ** 70) * 251] + [rng.randrange(-D * 4, D * 4) for _ in range(60)]
    nums += [rng.getrandbits(2000) * 3 ** 4 * 2 ** 3 for _ in range(20)]
    got = S.to_fractions(nums, D)
    assert got == [Fraction(v, D) for v in nums]
    assert all(math.gcd(f.numerator, f.denominator) == 1 and f.denominator > 0 for f in got)


def test_reduced_fraction_constructor_fallback():
    """Where Fraction has no ``_normalize`` argument the plain constructor
    serves (same value for inputs in lowest terms); where it has one, the
    unnormalised construction gives the same Fraction."""
    class NoNormalize(Fraction):
        def __new__(cls, numerator=0, denominator=None):
            return super().__new__(cls, numerator, denominator)

    assert S._make_reduced(NoNormalize) is NoNormalize
    make = S._make_reduced()
    for n, d in [(3, 7), (-5, 12), (0, 1), (2 ** 200 + 1, 3 ** 90)]:
        assert make(n, d) == Fraction(n, d)


def test_to_fractions_without_the_native_stage(monkeypatch):
    """The pure-Python branch of to_fractions (no GMP on the host) normalises
    like Fraction itself."""
    monkeypatch.setattr(S, "host_bigint_available", lambda: False)
    D = 2 ** 5 * 3 ** 3 * 251
    nums = [0, 1, -1, D, -2 * D, 6, -(2 ** 70) * 251, 12345]
    assert S.to_fractions(nums, D) == [Fraction(v, D) for v in nums]


def test_python_rational_reconstruction_against_the_oracle():
    """The pure-Python extended Euclid (used when GMP is missing) against the
    oracle's rational reconstruction, found and not-found cases alike."""
    rng = random.Random(12)
    M = O.prod([q for q in O.primes_largest_first() if q % 2][:8]) ** 3
    for _ in range(200):
        a, d = rng.randrange(-2 ** 40, 2 ** 40), rng.randrange(1, 2 ** 40)
        if math.gcd(a, d) != 1 or math.gcd(d, M) != 1:
            continue
        u = a * pow(d, -1, M) % M
        assert S._ratrec(u, M, 2 ** 40, 2 ** 40) == D.rational_reconstruct(u, M, 2 ** 40, 2 ** 40) == Fraction(a, d)
        v = rng.randrange(M)
        assert S._ratrec(v, M, 2 ** 20, 2 ** 20) == D.rational_reconstruct(v, M, 2 ** 20, 2 ** 20)
