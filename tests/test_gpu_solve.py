"""Parity of the Dixon-lift path (batched modular inverse, lift steps, exact
solve) with the oracle (oracle/dixon.py) (GPU only).

Cases follow exact-solve, "Correctness": bitwise against an exact Fraction
Gaussian elimination on small systems, a planted integer solution, a scaled
Hilbert system with dense denominators, the order-30 Pascal system, and the
integer identity A @ N == d * b at a larger size.
"""
import math
import random
from fractions import Fraction

import numpy as np
import pytest
import torch

import exact_integer_gemm_amd as rg
from exact_integer_gemm_amd.exact_solve import ODD_PRIMES
from oracle import dixon as D

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _setup():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    rg.load()
    yield


def dev(x):
    return torch.from_numpy(np.ascontiguousarray(np.asarray(x, dtype=np.int64))).cuda()


def _system(seed, n, c, amax, bmax):
    rng = random.Random(seed)
    A = [[rng.randint(-amax, amax) for _ in range(n)] for _ in range(n)]
    b = [[rng.randint(-bmax, bmax) for _ in range(c)] for _ in range(n)]
    return A, b


def test_batched_inverse_matches_oracle():
    """Inverses mod all 53 odd primes, with A singular mod 3 and mod 7."""
    n = 37
    A, _ = _system(1, n, 1, 1000, 1)
    A[0] = [21 * v for v in A[0]]          # det A becomes a multiple of 3 and 7
    print(f"batched inverse n={n}", flush=True)
    singular, ws = rg.batched_inverse(dev(A))
    sing = singular.cpu().tolist()
    for e, q in enumerate(ODD_PRIMES):
        assert bool(sing[e]) == (D.inverse_mod(A, q) is None), q
    assert sing[ODD_PRIMES.index(3)] and sing[ODD_PRIMES.index(7)]
    sel = [i for i, s in enumerate(sing) if not s]
    planes = rg.inverse_planes(ws, n, sel).cpu().numpy()
    for t in (0, 1, 2, len(sel) // 2, len(sel) - 1):
        q = ODD_PRIMES[sel[t]]
        ref = D.inverse_mod(A, q)
        ref_bal = [[v - q if v > q // 2 else v for v in row] for row in ref]
        assert np.array_equal(planes[t], np.array(ref_bal, dtype=np.int8)), q


@pytest.mark.parametrize("n,c", [(12, 3), (32, 1), (48, 4), (32, 5), (16, 2)])
def test_lift_digits_match_oracle(n, c):
    """n a multiple of 16 with at most 4 right-hand sides takes the fused step (digit and update
    kernels); the other shapes the batched residue product."""
    A, b = _system(2, n, c, 10 ** 6, 10 ** 6)
    singular, ws = rg.batched_inverse(dev(A))
    sel = [i for i, s in enumerate(singular.cpu().tolist()) if not s]
    moduli = [ODD_PRIMES[i] for i in sel]
    p = rg.plan_from_moduli(moduli, n)
    planes = rg.inverse_planes(ws, n, sel)
    digits = rg.dixon_lift(p, dev(A), dev(b), planes, 4).cpu().numpy()
    from oracle import oracle as O
    ref = D.dixon_digits(A, b, moduli, 4)
    for s in range(4):
        got = O.decode_array(digits[s])
        assert [[int(v) for v in row] for row in got] == ref[s], s


@pytest.mark.parametrize("n,c", [(1040, 1), (2064, 2)])
def test_lift_digits_large_p_adic_identity(n, c):
    """The fused lift where a row's work is spread over two waves (up to 2048 rows) or one: its first
    three digits x_s (balanced, |x_s| < P/2) satisfy A (x_0 + x_1 P + x_2 P^2) = b mod P^3, checked
    mod q^3 for every prime q of P (P^3 divides v exactly when every q^3 does), which fixes the
    balanced digits uniquely."""
    from oracle import oracle as O
    rng = np.random.default_rng(n)
    A = rng.integers(-2 ** 15, 2 ** 15, size=(n, n))
    b = rng.integers(-2 ** 15, 2 ** 15, size=(n, c))
    print(f"lift digits n={n} c={c}", flush=True)
    singular, ws = rg.batched_inverse(dev(A))
    sel = [i for i, s_ in enumerate(singular.cpu().tolist()) if not s_]
    moduli = [ODD_PRIMES[i] for i in sel]
    P = math.prod(moduli)
    p = rg.plan_from_moduli(moduli, n)
    planes = rg.inverse_planes(ws, n, sel)
    del ws
    digits = rg.dixon_lift(p, dev(A), dev(b), planes, 3).cpu().numpy()
    xs = [O.decode_array(digits[s_]) for s_ in range(3)]          # [n][c] Python ints per step
    for s_ in range(3):
        assert all(abs(int(v)) < P // 2 + 1 for row in xs[s_] for v in row)
    for q in moduli:
        qk = q ** 3
        X = np.array([[(int(xs[0][i][k]) + int(xs[1][i][k]) * P + int(xs[2][i][k]) * P * P) % qk
                       for k in range(c)] for i in range(n)], dtype=np.int64)
        # A X mod q^3 from two float64 products of 12-bit halves of X (sums below 2^47: exact)
        Af = (A % qk).astype(np.float64)
        lo = (Af @ (X & 4095).astype(np.float64)).astype(np.int64)
        hi = (Af @ (X >> 12).astype(np.float64)).astype(np.int64)
        res = ((hi % qk) * 4096 + lo - b) % qk
        assert not res.any(), q


@pytest.mark.parametrize("seed,n,c", [(3, 5, 1), (4, 16, 3), (5, 40, 2), (6, 1, 1)])
def test_solve_matches_fraction_elimination(seed, n, c):
    print(f"solve n={n} c={c}", flush=True)
    A, b = _system(seed, n, c, 1000, 1000)
    X = rg.solve(dev(A), dev(b))
    assert X == D.solve_fraction(A, b)


def test_planted_integer_solution():
    n = 128
    rng = np.random.default_rng(7)
    A = rng.integers(-2 ** 23, 2 ** 23, size=(n, n))
    x = rng.integers(-10 ** 6, 10 ** 6, size=(n, 1))
    b = A @ x
    print(f"planted n={n}", flush=True)
    X, info = rg.solve(dev(A), dev(b), return_info=True)
    assert info["denominator"] == 1
    assert [[int(v) for v in row] for row in X] == x.tolist()


def test_scaled_hilbert_dense_denominators():
    n = 9
    L = math.lcm(*range(1, 2 * n))
    A = [[L // (i + j + 1) for j in range(n)] for i in range(n)]
    b = [[1], [0], [-1], [2], [0], [3], [1], [-2], [5]]
    X = rg.solve(dev(A), dev(b))
    assert X == D.solve_fraction(A, b)
    assert max(v[0].denominator for v in X) > 1


def test_pascal_order_30():
    """The page's example: the order-30 Pascal matrix is unimodular, so the
    solution is integral; A x == b in integer arithmetic."""
    n = 30
    A = [[math.comb(i + j, i) for j in range(n)] for i in range(n)]
    rng = random.Random(8)
    b = [[rng.randint(-10 ** 6, 10 ** 6)] for _ in range(n)]
    X = rg.solve(dev(A), dev(b))
    assert all(v[0].denominator == 1 for v in X)
    xs = [int(v[0]) for v in X]
    assert [sum(A[i][j] * xs[j] for j in range(n)) for i in range(n)] == [r[0] for r in b]


def test_singular_system():
    A, b = _system(9, 10, 1, 100, 100)
    A[9] = [A[0][j] - 3 * A[4][j] for j in range(10)]
    assert rg.solve(dev(A), dev(b)) is None


def test_identity_at_larger_size():
    """n = 256, 24-bit entries, two right-hand sides: A @ N == d * b."""
    n, c = 256, 2
    rng = np.random.default_rng(10)
    A = rng.integers(-2 ** 23, 2 ** 23, size=(n, n))
    b = rng.integers(-2 ** 23, 2 ** 23, size=(n, c))
    print(f"identity n={n}", flush=True)
    X, info = rg.solve(dev(A), dev(b), return_info=True)
    d = info["denominator"]
    N = np.array(info["numerators"], dtype=object).reshape(n, c)
    AN = A.astype(object).dot(N)
    assert np.array_equal(AN, d * b.astype(object))
    assert d > 1


def test_lift_rejects_even_modulus():
    p = rg.plan_n(3)               # 251, 241, 239: odd, accepted
    A = dev(np.eye(4, dtype=np.int64))
    b = dev(np.ones((4, 1), dtype=np.int64))
    planes = torch.zeros((3, 4, 4), dtype=torch.int8, device="cuda")
    rg.dixon_lift(p, A, b, planes, 1)
    p2 = rg.plan_from_moduli([256, 251], 4)
    with pytest.raises(rg.RnsError) as e:
        rg.dixon_lift(p2, A, b, torch.zeros((2, 4, 4), dtype=torch.int8, device="cuda"), 1)
    assert e.value.code == -1


def test_nonsingular_but_singular_mod_every_prime():
    """det A is a multiple of all 53 odd primes below 256 yet nonzero: the lift has no prime left,
    and the solve must raise rather than report a singular system."""
    n = 10
    groups, cur = [], 1
    for q in ODD_PRIMES:
        if cur * q * n >= 1 << 62:
            groups.append(cur)
            cur = 1
        cur *= q
    groups.append(cur)
    assert len(groups) <= n
    diag = groups + [1] * (n - len(groups))
    A = np.diag(np.array(diag, dtype=np.int64))
    b = np.ones((n, 1), dtype=np.int64)
    with pytest.raises(rg.RnsError) as e:
        rg.solve(dev(A), dev(b))
    assert e.value.code == -3


def _planted_lu(n, seed, diag_factor_rows):
    """A = L U with L unit lower triangular (entries in {-1, 0, 1}) and U upper triangular with
    entries in [-3, 3]: det A = prod(diag U), so A is singular exactly mod the primes dividing
    some diagonal entry.  diag_factor_rows: {row: diagonal value}."""
    rng = np.random.default_rng(seed)
    L = np.tril(rng.integers(-1, 2, size=(n, n)), -1) + np.eye(n, dtype=np.int64)
    U = np.triu(rng.integers(-3, 4, size=(n, n)), 1) + np.eye(n, dtype=np.int64)
    for r, v in diag_factor_rows.items():
        U[r, r] = v
    return (L.astype(np.float64) @ U.astype(np.float64)).astype(np.int64)   # exact: |sums| < 2^53


def _check_inverses(A, planes, sel, primes_to_check):
    Af = A.astype(np.float64)
    n = A.shape[0]
    for t in primes_to_check:
        q = ODD_PRIMES[sel[t]]
        Bq = planes[t].astype(np.float64)
        prod = np.mod(np.mod(Af, q) @ Bq, q)     # exact: n * 255 * 127 < 2^53
        assert np.array_equal(prod, np.eye(n)), q


@pytest.mark.parametrize("n", [300, 2100, 4097])
def test_batched_inverse_larger_sizes(n):
    """The blocked elimination (panels of 32 columns up to 2048 rows, 16 up to 4096, ragged last
    panel) and the unblocked one above 4096: A B = I mod q, and the singular flags match the
    planted determinant (diagonal entries 3 * 7 and 5 * 11)."""
    A = _planted_lu(n, 11 + n, {n // 3: 21, n - 1: 55})
    print(f"batched inverse n={n}", flush=True)
    singular, ws = rg.batched_inverse(dev(A))
    sing = singular.cpu().tolist()
    assert [ODD_PRIMES[e] for e, s in enumerate(sing) if s] == [11, 7, 5, 3]
    sel = [i for i, s in enumerate(sing) if not s]
    planes = rg.inverse_planes(ws, n, sel).cpu().numpy()
    _check_inverses(A, planes, sel, (0, len(sel) - 1) if n > 4096 else (0, 1, len(sel) // 2, len(sel) - 1))


def test_empty_and_degenerate_shapes():
    assert rg.solve(dev(np.zeros((0, 0))), dev(np.zeros((0, 1)))) == []
    with pytest.raises(ValueError):
        rg.solve(dev(np.eye(3)), dev(np.zeros((3, 0))))
    X = rg.solve(dev([[7]]), dev([[3, -14]]))          # 1 x 1, two right-hand sides
    assert X == [[Fraction(3, 7), Fraction(-2)]]


@pytest.mark.parametrize("n_primes,m,count", [(3, 4, 70), (20, 7, 130), (50, 11, 64), (53, 3, 1)])
def test_padic_chunks_match_the_oracle(n_primes, m, count):
    """The p-adic values in binary (two exact residue products and a carry pass) against the
    oracle's sum of digits times powers of P, for one- to six-limb digits."""
    from oracle import oracle as O
    rng = np.random.default_rng(20 + n_primes)
    ps = ODD_PRIMES[:n_primes]
    P = math.prod(ps)
    L = (P.bit_length() + 64) // 64
    vals = [[int(v) for v in rng.integers(-(P // 2), P // 2, size=count, dtype=np.int64)] if P < 2 ** 62 else
            [int.from_bytes(rng.bytes((P.bit_length() + 7) // 8), "little") % P - P // 2 for _ in range(count)]
            for _ in range(m)]
    dig = np.zeros((m, count, L), dtype=np.int64)
    for s in range(m):
        for i in range(count):
            dig[s, i] = O.to_limbs(vals[s][i], L)
    print(f"padic chunks primes={n_primes} m={m} count={count}", flush=True)
    chunks = rg.exact_solve.padic_chunks(dev(dig), P, m).cpu().numpy().view(np.uint32)
    T = chunks.shape[1]
    ref = D.padic_value([[[v] for v in row] for row in vals], P)
    for i in range(count):
        got = int.from_bytes(chunks[i].tobytes(), "little", signed=True)
        assert got == ref[i][0], i
    assert 32 * T > (P ** m).bit_length()
    # the operand layout: int64 [T][count] chunk values, the top one signed
    cols = rg.exact_solve.padic_chunks(dev(dig), P, m, transposed=True).cpu().numpy()
    assert cols.shape == (T, count)
    assert np.array_equal(cols[:-1].T.astype(np.uint32), chunks[:, :-1])
    assert np.array_equal(cols[-1], chunks[:, -1].view(np.int32).astype(np.int64))


@pytest.mark.parametrize("n_primes,m,count,dbits", [(3, 6, 70, 50), (20, 9, 130, 700), (50, 12, 65, 2500),
                                                    (53, 4, 1, 10)])
def test_chunk_modmul_is_d_times_x_mod_pm(n_primes, m, count, dbits):
    """The GPU's one modular multiply per numerator: (D X - q P^m) mod 2^(32 Tw) equal to the Barrett
    step written out in Python integers, congruent to D X mod P^m and below P^m in magnitude, for
    balanced p-adic values (extremes included) and denominators up to the bound."""
    from oracle import oracle as O
    rng = random.Random(n_primes + m)
    P = math.prod(ODD_PRIMES[:n_primes])
    Pm = P ** m
    half = (Pm - 1) // 2
    Db = (1 << dbits) - 1
    L = (P.bit_length() + 64) // 64
    vals = [[rng.randrange(-(P // 2), P // 2 + 1) for _ in range(count)] for _ in range(m)]
    vals[m - 1][0] = P // 2                             # the largest value, then its negative
    if count > 1:
        vals[m - 1][1] = -(P // 2)
    dig = np.zeros((m, count, L), dtype=np.int64)
    for s_ in range(m):
        for i in range(count):
            dig[s_, i] = O.to_limbs(vals[s_][i], L)
    X = D.padic_value([[[v] for v in row] for row in vals], P)
    consts = rg.exact_solve.ModmulConstants(P, m, Db, torch.device("cuda", 0))
    mu = sum(int(v) << (32 * i) for i, v in enumerate(consts.mu.cpu().tolist()))
    Xt = rg.exact_solve.padic_chunks(dev(dig), P, m, transposed=True)
    for Dv in (Db, rng.randrange(1, Db), 1):
        print(f"chunk modmul primes={n_primes} m={m} count={count} D bits={Dv.bit_length()}", flush=True)
        w0 = rg.exact_solve.chunk_modmul(Xt, Dv, consts).cpu().numpy().view(np.uint32)
        assert w0.shape == (count, consts.Tw)
        for i in range(count):
            got = int.from_bytes(w0[i].tobytes(), "little", signed=True)
            x = X[i][0]
            assert abs(x) <= half
            Y = Dv * x
            q = ((Y >> (32 * consts.s1c)) * mu + (1 << (32 * consts.k2c - 1))) >> (32 * consts.k2c)
            assert got == Y - q * Pm, (Dv.bit_length(), i)
            assert (got - Y) % Pm == 0 and abs(got) < Pm


@pytest.mark.parametrize("Tw,bbits", [(5, 70), (40, 1000), (300, 5000), (3, 94)])
def test_chunk_bound_edges(Tw, bbits):
    """The numerators' bound test: ok exactly when |w| <= B, at B, B + 1, -B, -B - 1, 0, -1, the
    extremes of Tw chunks and random values; the numerator's limbs when ok, zeros otherwise."""
    rng = random.Random(Tw)
    B = rng.getrandbits(bbits) | (1 << (bbits - 1))
    top = 2 ** (32 * Tw - 1)
    vals = [B, B + 1, -B, -B - 1, 0, -1, 1, top - 1, -top, B - 1, -(B - 1)]
    vals += [rng.randrange(-B, B + 1) for _ in range(40)] + [rng.randrange(-top, top) for _ in range(20)]
    vals += [rng.choice([-1, 1]) * (B + rng.randrange(1, 2 ** 40)) for _ in range(10)]
    w = np.zeros((len(vals), Tw), dtype=np.uint32)
    for i, v in enumerate(vals):
        w[i] = np.frombuffer((v % (1 << (32 * Tw))).to_bytes(4 * Tw, "little"), dtype=np.uint32)
    print(f"chunk bound Tw={Tw} B bits={bbits}", flush=True)
    ok, num, used = rg.exact_solve.chunk_bound(torch.from_numpy(w.view(np.int32)).cuda(), B)
    ok = ok.cpu().numpy()
    num = num.cpu().numpy()
    used = used.cpu().numpy()
    wl = num.shape[1]
    assert wl * 64 > bbits
    for i, v in enumerate(vals):
        assert bool(ok[i]) == (abs(v) <= B), (i, v)
        got = int.from_bytes(num[i].tobytes(), "little", signed=True)
        assert got == (v if abs(v) <= B else 0), i
        if ok[i]:
            # the reported limbs hold the value with its sign, and no more than w_limbs
            assert 1 <= used[i] <= wl and v.bit_length() < 64 * used[i], (i, used[i])
            assert int.from_bytes(num[i, :used[i]].tobytes(), "little", signed=True) == v
        else:
            assert used[i] == 0
