"""Pins of the CPU oracle against facts the pages and mathematics fix.

None of these tests needs a GPU.  Each pin is chosen so that a plausible slip
in the oracle (a dropped term, a wrong sign or index, an off-by-one in a
bound, a transposed operand) fails at least one of them; the checks compare
against library routines (sympy, numpy object arithmetic), closed forms,
brute force or figures printed on the pages (tests/golden/pages_constants.json).
"""
import itertools
import json
import math
import os

import numpy as np
import pytest
import sympy
from sympy.ntheory.modular import crt as sympy_crt

from oracle import oracle as O
from oracle import cgemm

GOLD = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "pages_constants.json")))


# --------------------------------------------------------------------------
# prime table and capacity
# --------------------------------------------------------------------------
def test_primes_match_sympy():
    assert O.primes_below(256) == list(sympy.primerange(2, 256))
    assert len(O.primes_below(256)) == 54
    ps = O.primes_largest_first()
    assert ps[:4] == [251, 241, 239, 233] and ps[-1] == 2


def test_product_is_335_bit():
    # enclosure-gemm, Requirements and limits: "335-bit product of the primes below 256"
    P = O.prod(O.primes_below(256))
    assert P.bit_length() == GOLD["product_of_primes_below_256_bits"]["value"]
    assert P == sympy.primorial(54)


def test_362_8_bits_is_a_different_modulus_set():
    # Ozaki paper §1.2 / §4.2.2 quote a 362.8-bit INT8 capacity; that is the
    # product of the largest prime powers <= 256 (lcm(1..256)), not of the
    # primes, which is why the 335-bit figure is the one built on.
    lcm = 1
    for i in range(1, 257):
        lcm = lcm * i // math.gcd(lcm, i)
    assert round(math.log2(lcm), 1) == GOLD["int8_crt_capacity_bits"]["value"]
    assert math.log2(O.prod(O.primes_below(256))) < 335


def test_int32_accumulator_bound():
    # K <= 2^17 (both pages): with balanced residues |r| <= 125 for q = 251 the
    # int32 accumulator cannot overflow, and 2^17 is the largest power of two
    # for which that holds.
    assert O.K_MAX == GOLD["k_max"]["value"]
    rmax = max(abs(O.balanced(x, q)) for q in O.primes_below(256) for x in range(q))
    assert rmax == 125
    assert O.K_MAX * rmax * rmax < 2 ** 31
    assert 2 * O.K_MAX * rmax * rmax >= 2 ** 31
    # a residue plane read as any int8 value (batched-residue step) times a
    # balanced residue still fits
    assert O.K_MAX * 128 * 125 < 2 ** 31


@pytest.mark.parametrize("K,a,b,n", [(64, 20, 20, 6), (1024, 31, 31, 10),
                                     (4096, 55, 55, 16), (4096, 100, 100, 29)])
def test_prime_count_for_the_workloads(K, a, b, n):
    # Independent route: compare the bound with sums of float logs of sympy's
    # primes (the margins below are far larger than float error).
    logs = [math.log2(p) for p in sorted(sympy.primerange(2, 256), reverse=True)]
    need = 1 + math.log2(K) + a + b
    assert sum(logs[:n]) > need + 1e-9
    assert sum(logs[:n - 1]) < need - 1e-9
    assert len(O.prime_set_for_bound(K, a, b)) == n


def test_capacity_budget_from_the_pages_is_accepted():
    # enclosure-gemm, Requirements and limits: bits_a + bits_b + ceil(log2 K) <= 332
    budget = GOLD["capacity_budget_bits"]["value"]
    for K in (1, 2, 3, 1000, 4096, 2 ** 17):
        lk = math.ceil(math.log2(K)) if K > 1 else 0
        a = (budget - lk) // 2
        b = budget - lk - a
        ps = O.prime_set_for_bound(K, a, b)
        assert O.prod(ps) > 2 * K * 2 ** (a + b)
    with pytest.raises(ValueError):
        O.prime_set_for_bound(4096, 170, 170)
    with pytest.raises(ValueError):
        O.prime_set_for_bound(2 ** 17 + 1, 1, 1)


def test_limbs_to_hold():
    # (-P/2, P/2] for the 54-prime P needs 335 bits: six limbs (the pages'
    # signed 384-bit Garner word is exactly six limbs)
    P = O.prod(O.primes_below(256))
    assert O.limbs_to_hold(P) * 64 == GOLD["garner_word_bits"]["value"]
    assert O.limbs_to_hold(251) == 1
    assert O.limbs_to_hold(2 ** 64 - 1) == 1 and O.limbs_to_hold(2 ** 64 + 1) == 2


# --------------------------------------------------------------------------
# limbs
# --------------------------------------------------------------------------
def test_limb_constants():
    assert O.to_limbs(-1, 1) == [-1]
    assert O.to_limbs(-1, 3) == [-1, -1, -1]
    assert O.to_limbs(2 ** 64, 2) == [0, 1]
    assert O.to_limbs(-(2 ** 64), 2) == [0, -1]
    assert O.to_limbs(2 ** 127 - 1, 2) == [-1, 2 ** 63 - 1]
    assert O.to_limbs(-(2 ** 127), 2) == [0, -(2 ** 63)]
    assert O.to_limbs(2 ** 63, 2) == [-(2 ** 63), 0]
    with pytest.raises(OverflowError):
        O.to_limbs(2 ** 63, 1)
    rng = np.random.default_rng(0)
    for L in (1, 2, 3, 4, 6):
        for _ in range(200):
            x = int(rng.integers(-(1 << 62), 1 << 62)) << int(rng.integers(0, 64 * L - 63))
            assert O.from_limbs(O.to_limbs(x, L)) == x


def test_decode_encode_arrays():
    vals = np.array([[0, -1, 2 ** 100, -(2 ** 100)], [5, -5, 2 ** 127 - 1, -(2 ** 127)]], dtype=object)
    enc = O.encode_array(vals, 2)
    assert enc.dtype == np.int64 and enc.shape == (2, 4, 2)
    assert np.all(O.decode_array(enc) == vals)
    # byte-level check of one entry against Python's own two's-complement bytes
    x = -(2 ** 100) + 12345
    assert enc.shape[-1] == 2
    raw = O.encode_array(np.array([x], dtype=object), 2).tobytes()
    assert raw == x.to_bytes(16, "little", signed=True)


# --------------------------------------------------------------------------
# balanced residues
# --------------------------------------------------------------------------
def test_balanced_exhaustive_int16():
    xs = np.arange(-(1 << 15), 1 << 15)
    for q in O.primes_below(256):
        h = (q - 1) // 2
        r = O.balanced_array(xs, q)
        assert np.all(np.mod(xs - r, q) == 0)
        assert r.min() >= -h and r.max() <= q // 2
        # an independent formula: shift into [0, q), reduce, shift back
        assert np.array_equal(r, np.mod(xs + h, q) - h)
    assert [O.balanced(x, 2) for x in (-3, -2, -1, 0, 1, 2)] == [1, 0, 1, 0, 1, 0]


def test_balanced_edge_limbs():
    edge = [0, 1, -1, 2 ** 63 - 1, -(2 ** 63), 2 ** 64 - 1, 2 ** 64, -(2 ** 127), 2 ** 127 - 1]
    for q in (2, 3, 5, 127, 251):
        for x in edge:
            r = O.balanced(x, q)
            assert (x - r) % q == 0 and -(q - 1) // 2 <= r <= q // 2


# --------------------------------------------------------------------------
# reconstruction
# --------------------------------------------------------------------------
def test_crt_round_trip_and_sympy():
    rng = np.random.default_rng(7)
    for n in (1, 2, 6, 10, 29, 53, 54):
        ps = O.primes_largest_first()[:n]
        P = O.prod(ps)
        for _ in range(50):
            X = int.from_bytes(rng.bytes(48), "little") % P - P // 2
            if 2 * X <= -P:
                X += P
            res = [X % q for q in ps]
            assert O.crt_balanced(res, ps) == X
            v, m = sympy_crt(ps, res)
            assert m == P
            v = int(v)
            assert (v - P if 2 * v > P else v) == X


def test_crt_boundaries():
    for ps in (O.primes_largest_first()[:6], O.primes_largest_first()):  # odd P, even P
        P = O.prod(ps)
        if P % 2:
            cases = [0, 1, -1, (P - 1) // 2, -(P - 1) // 2]
        else:
            cases = [0, 1, -1, P // 2, -P // 2 + 1]
        for X in cases:
            assert O.crt_balanced([X % q for q in ps], ps) == X
        # just outside the range wraps to the other end
        top = P // 2
        assert O.crt_balanced([(top + 1) % q for q in ps], ps) == top + 1 - P


def test_crt_rounded_quotient_against_sympy():
    """Ozaki II §3.5.2 reading (rounded quotient) against sympy's CRT, both P
    parities, random values and the ends of (-P/2, P/2]."""
    rng = np.random.default_rng(17)
    for n in (1, 6, 16, 29, 53, 54):
        ps = O.primes_largest_first()[:n]
        P = O.prod(ps)
        ends = [0, 1, -1, P // 2, -((P - 1) // 2)]
        vals = ends + [int.from_bytes(rng.bytes(48), "little") % P - P // 2 for _ in range(40)]
        for X in vals:
            if 2 * X <= -P:
                X += P
            res = [X % q for q in ps]
            v, m = sympy_crt(ps, res)
            v = int(v)
            want = v - P if 2 * v > P else v
            assert want == X
            assert O.crt_rounded_quotient(res, ps) == X


def test_crt_rounded_quotient_off_by_one_estimates():
    """Any quotient estimate within one of the true one gives the same value
    (the exact comparison with P/2 repairs it); one two away does not, so the
    repair is a single step and not a hidden second reduction."""
    ps = O.primes_largest_first()
    P = O.prod(ps)
    rng = np.random.default_rng(23)
    for X in [P // 2, -(P // 2) + 1, 0, 5] + [int.from_bytes(rng.bytes(48), "little") % P - P // 2
                                            for _ in range(20)]:
        res = [X % q for q in ps]
        u = [O.balanced(r * pow(P // q, -1, q), q) for r, q in zip(res, ps)]
        S = sum(uj * (P // q) for uj, q in zip(u, ps))
        t_true = (S - X) // P
        assert (S - X) % P == 0
        for d in (-1, 0, 1):
            assert O.crt_rounded_quotient(res, ps, lambda u_, p_: t_true + d) == X
        assert O.crt_rounded_quotient(res, ps, lambda u_, p_: t_true + 2) != X
    # a binary64 estimate of sum u_j / q_j, rounded to nearest, is one such estimate
    for X in (P // 2, -(P // 2) + 1, 12345):
        res = [X % q for q in ps]
        est = lambda u_, p_: round(sum(float(a) / float(b) for a, b in zip(u_, p_)))
        assert O.crt_rounded_quotient(res, ps, est) == X


def test_garner_digits_against_crt():
    rng = np.random.default_rng(11)
    odd = O.primes_largest_first()[:53]
    two_first = [2] + odd
    two_last = odd + [2]
    for ps in (odd[:10], odd[:29], odd, two_first):
        P = O.prod(ps)
        for _ in range(30):
            X = int.from_bytes(rng.bytes(48), "little") % P - P // 2
            if 2 * X <= -P:
                X += P
            res = [O.balanced(X, q) for q in ps]
            d = O.garner_digits(res, ps)
            assert all(-(q - 1) // 2 <= di <= q // 2 for di, q in zip(d, ps))
            assert O.mixed_radix_value(d, ps) == O.crt_balanced(res, ps) == X
    # with 2 last, balanced digits can land one period above (-P/2, P/2]:
    # X = (P/2 - 1)/2 + P/2 has the top digit 1 and is congruent but too big
    P = O.prod(two_last)
    Xhi = (P // 2 - 1) // 2 + P // 2
    res = [Xhi % q for q in two_last]
    val = O.mixed_radix_value(O.garner_digits(res, two_last), two_last)
    assert val == Xhi and 2 * val > P and O.crt_balanced(res, two_last) == Xhi - P


# --------------------------------------------------------------------------
# the integer product
# --------------------------------------------------------------------------
def test_int_matmul_brute_force_tiny():
    vals = [-2, -1, 0, 1, 2]
    for M, K, N in [(1, 1, 1), (1, 2, 1), (2, 1, 2), (2, 2, 2)]:
        for flat in itertools.islice(itertools.product(vals, repeat=M * K + K * N), 0, None, 97):
            A = np.array(flat[:M * K], dtype=object).reshape(M, K)
            B = np.array(flat[M * K:], dtype=object).reshape(K, N)
            assert np.array_equal(np.array(O.int_matmul(A.tolist(), B.tolist()), dtype=object), A.dot(B))


def test_int_matmul_closed_forms():
    K = 5
    I = [[int(i == j) for j in range(K)] for i in range(K)]
    B = [[(-1) ** (i + j) * (2 ** 90 + i * 7 + j) for j in range(3)] for i in range(K)]
    assert O.int_matmul(I, B) == B
    a, b = 100, 100
    A = [[-(2 ** a)] * K]
    Bm = [[-(2 ** b)] for _ in range(K)]
    assert O.int_matmul(A, Bm) == [[K * 2 ** (a + b)]]
    alt = [[(-1) ** k for k in range(4)]]
    ones = [[1] for _ in range(4)]
    assert O.int_matmul(alt, ones) == [[0]]
    # non-square shapes keep A's rows and B's columns (a transposed operand fails)
    A = [[1, 2, 3]]
    B = [[1], [10], [100]]
    assert O.int_matmul(A, B) == [[321]]
    assert O.int_matmul(B, A) == [[1, 2, 3], [10, 20, 30], [100, 200, 300]]


@pytest.fixture(scope="module")
def cg():
    cgemm.build()
    return cgemm


@pytest.mark.parametrize("la,lb,abits,bbits", [(1, 1, 20, 20), (1, 1, 62, 62), (2, 2, 100, 100),
                                               (1, 2, 40, 120), (3, 1, 180, 50), (4, 4, 250, 250)])
def test_c_oracle_matches_python(cg, la, lb, abits, bbits):
    from workloads import random_operands
    M, N, K = 7, 5, 9
    A, B = random_operands(100 + la * 10 + lb, M, N, K, la, lb, abits, bbits)
    Av, Bv = O.decode_array(A), O.decode_array(B)
    ref = np.array(O.int_matmul(Av.tolist(), Bv.tolist()), dtype=object)
    lc = O.limbs_to_hold(2 * K * 2 ** (abits + bbits) + 1) + 1
    C = cg.gemm(A, B, lc)
    assert np.array_equal(O.decode_array(C), ref)


def test_c_oracle_extremes(cg):
    # the most negative L-limb values: magnitude 2^(64L-1), products hit the top bits
    for L in (1, 2, 4):
        lo = -(2 ** (64 * L - 1))
        hi = 2 ** (64 * L - 1) - 1
        A = O.encode_array(np.array([[lo, hi, lo, -1]], dtype=object), L)
        B = O.encode_array(np.array([[lo], [lo], [hi], [1]], dtype=object), L)
        ref = lo * lo + hi * lo + lo * hi - 1
        C = cg.gemm(A, B, 2 * L + 1)
        assert O.decode_array(C)[0, 0] == ref
    # overflow is reported, not hidden
    A = O.encode_array(np.array([[2 ** 62, 2 ** 62]], dtype=object), 1)
    B = O.encode_array(np.array([[2], [2]], dtype=object), 1)
    with pytest.raises(OverflowError):
        cg.gemm(A, B, 1)
    assert O.decode_array(cg.gemm(A, B, 2))[0, 0] == 2 ** 64


def test_c_oracle_empty_and_k0(cg):
    A = np.zeros((3, 0, 1), dtype=np.int64)
    B = np.zeros((0, 4, 1), dtype=np.int64)
    C = cg.gemm(A, B, 2)
    assert C.shape == (3, 4, 2) and not C.any()
    A = np.zeros((0, 5, 1), dtype=np.int64)
    B = np.zeros((5, 4, 1), dtype=np.int64)
    assert cg.gemm(A, B, 1).shape == (0, 4, 1)


def test_c_oracle_freivalds_medium(cg):
    from workloads import random_operands
    M, N, K = 96, 80, 200
    A, B = random_operands(5, M, N, K, 2, 2, 100, 100)
    C = cg.gemm(A, B, 4)
    Av, Bv, Cv = O.decode_array(A), O.decode_array(B), O.decode_array(C)
    rng = np.random.default_rng(3)
    for _ in range(2):
        v = rng.integers(-(1 << 16), 1 << 16, size=N, endpoint=True)
        assert O.freivalds_holds(Av, Bv, Cv, v)
    # a single wrong entry is caught
    Cbad = Cv.copy()
    Cbad[17, 33] += 1
    v = rng.integers(-(1 << 16), 1 << 16, size=N, endpoint=True)
    assert not O.freivalds_holds(Av, Bv, Cbad, v)


# --------------------------------------------------------------------------
# stage definitions
# --------------------------------------------------------------------------
def test_residue_path_reproduces_the_integer_product():
    # The method's own steps (residues, one product per prime, CRT) must give
    # the integer product whenever P > 2 max|C| (exact-solve, Method;
    # Ozaki paper §3.1).
    from workloads import random_operands
    M, N, K = 6, 5, 8
    A, B = random_operands(9, M, N, K, 2, 2, 90, 90)
    Av, Bv = O.decode_array(A), O.decode_array(B)
    ps = O.prime_set_for_bound(K, 90, 90)
    Ares = O.residue_planes(Av, ps)
    Bres = O.residue_planes(Bv, ps)
    Y = [O.residue_product(Ares[j], Bres[j], q) for j, q in enumerate(ps)]
    X = O.crt_balanced_array(Y, ps)
    assert np.array_equal(X, Av.dot(Bv))
    # and the batched-residue step on the same planes gives the same result
    assert np.array_equal(O.residue_gemm_via_crt(Ares, Bv, ps), Av.dot(Bv))
    # one prime short is not enough for the extreme entry
    Aext = np.full((1, K), -(2 ** 90), dtype=object)
    Bext = np.full((K, 1), -(2 ** 90), dtype=object)
    short = ps[:-1]
    if O.prod(short) <= 2 * K * 2 ** 180:
        Ys = [O.residue_product(O.residue_planes(Aext, short)[j], O.residue_planes(Bext, short)[j], q)
              for j, q in enumerate(short)]
        assert O.crt_balanced_array(Ys, short)[0, 0] != K * 2 ** 180


def test_batched_residue_step_invariants():
    rng = np.random.default_rng(21)
    ps = O.primes_largest_first()
    from workloads import balanced_residue_planes
    M, K, N = 12, 10, 3
    Ares = balanced_residue_planes(rng, ps, M, K)
    r = rng.integers(-(1 << 34), 1 << 34, size=(K, N), endpoint=True)
    X = O.residue_gemm_via_crt(Ares, r, ps)
    P = O.prod(ps)
    v = rng.integers(-50, 50, size=N)
    for j, q in enumerate(ps):
        # X = Ares_j @ r (mod q_j) entrywise ...
        ref = np.mod(Ares[j].astype(object).dot(r.astype(object)), q)
        assert np.array_equal(np.mod(X, q), ref)
        # ... and the Freivalds-style identity holds mod q_j
        lhs = np.mod(X.dot(v.astype(object)), q)
        rhs = np.mod(Ares[j].astype(object).dot(r.astype(object).dot(v.astype(object))), q)
        assert np.array_equal(lhs, rhs)
    assert np.all(2 * X <= P) and np.all(2 * X > -P)


# ---------------------------------------------------------------------------
# prime-power moduli (Ozaki Scheme II paper, §1.2 / §4.2.2: 362.8-bit capacity)
# ---------------------------------------------------------------------------
def test_prime_power_moduli_product_is_lcm():
    import math as _m
    ms = O.prime_power_moduli()
    assert len(ms) == 54 and ms[0] == 256 and ms[2] == 243
    assert O.prod(ms) == _m.lcm(*range(1, 257))
    assert abs(_m.log2(O.prod(ms)) - 362.8) < 0.05
    for a in ms:
        for b in ms:
            assert a == b or _m.gcd(a, b) == 1


def test_moduli_set_for_bound_prime_powers():
    import math as _m
    ms = O.moduli_set_for_bound(4096, 170, 170, prime_powers=True)   # beyond the 335-bit primes
    assert O.prod(ms) > 2 * 4096 * 2 ** 340 and O.prod(ms[:-1]) <= 2 * 4096 * 2 ** 340
    with pytest.raises(ValueError):
        O.prime_set_for_bound(4096, 170, 170)
    with pytest.raises(ValueError):
        O.moduli_set_for_bound(2 ** 17, 1, 1, prime_powers=True)
    with pytest.raises(ValueError):
        O.moduli_set_for_bound(8, 180, 180, prime_powers=True)


def test_crt_with_prime_power_moduli():
    """CRT and Garner over the composite (coprime) moduli against sympy, at
    both ends of (-P/2, P/2] for the even P that contains 256."""
    from sympy.ntheory.modular import crt as sympy_crt
    rng = np.random.default_rng(31)
    ms = O.prime_power_moduli()[:12]
    P = O.prod(ms)
    for X in [0, 1, -1, P // 2, -(P // 2) + 1, P // 3, -(P // 7)] + [int(v) for v in rng.integers(-2 ** 62, 2 ** 62, 20)]:
        res = [O.balanced(X, q) for q in ms]
        assert O.crt_balanced(res, ms) == X
        assert O.crt_rounded_quotient(res, ms) == X
        r0, _ = sympy_crt(ms, [r % q for r, q in zip(res, ms)])
        assert (int(r0) - X) % P == 0
        assert O.mixed_radix_value(O.garner_digits(res, ms), ms) == X


# --------------------------------------------------------------------------
# stored digests of the five workloads (tests/golden/workload_digests.json)
# --------------------------------------------------------------------------
def _digests():
    return json.load(open(os.path.join(os.path.dirname(__file__), "golden", "workload_digests.json")))


def _sha(a):
    import hashlib
    return hashlib.sha256(np.ascontiguousarray(a).tobytes()).hexdigest()


def test_workload_digest_inputs():
    """The seeded generators still draw the inputs the digests were made from."""
    import workloads as W
    d = _digests()
    for name in W.NAMES:
        wl = W.make(name, primes=O.primes_largest_first()) if name == "dixon" else W.make(name)
        arrays = {"A_res": wl.A_res, "B": wl.B} if name == "dixon" else {"A": wl.A, "B": wl.B}
        for k, a in arrays.items():
            assert _sha(a) == d[name]["inputs_sha256"][k], (name, k)


@pytest.mark.parametrize("name", ["tiny", "dixon"])
def test_workload_digest_outputs_small(name):
    """The small digests recomputed by independent oracle routes: the tiny
    product by the Python triple loop, the batched step by Garner digits
    instead of the textbook CRT the digest script used."""
    import workloads as W
    d = _digests()[name]
    if name == "tiny":
        wl = W.make("tiny")
        C = O.int_matmul(O.decode_array(wl.A).tolist(), O.decode_array(wl.B).tolist())
        arr = O.encode_array(np.array(C, dtype=object), d["out_limbs"])
    else:
        primes = O.primes_largest_first()
        wl = W.make("dixon", primes=primes)
        # per-prime products mod q, then Garner with 2 first (range (-P/2, P/2])
        Y = [O.residue_product(wl.A_res[j].astype(np.int64), O.balanced_array(wl.B[..., 0], q), q)
             for j, q in enumerate(primes)]
        order = sorted(range(len(primes)), key=lambda j: primes[j] != 2)
        qs = [primes[j] for j in order]
        flat = [Y[j].ravel() for j in order]
        vals = [O.mixed_radix_value(O.garner_digits([int(f[e]) for f in flat], qs), qs) for e in range(flat[0].size)]
        arr = O.encode_array(np.array(vals, dtype=object).reshape(Y[0].shape), d["out_limbs"])
    assert _sha(arr) == d["C_sha256"]
