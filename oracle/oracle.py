"""Plain, slow, obviously-correct definitions for the exact residue GEMM.

TEST INFRASTRUCTURE ONLY: imported by the test suite, the smoke check and the
``cpu_baseline`` leg of ``bench.py``; never by the product path.

Everything here works on Python integers (or numpy ``object`` arrays holding
Python integers), so there is no overflow anywhere.  Each function names the
passage of the pages it follows:

* exact-solve, "Method": the modulus is a square-free product of primes below
  256, one INT8 product per prime, and balanced Garner reassembles the wide
  base-P digit; the precision must exceed twice the bound on the result.
* exact-solve, "Method" / "Requirements and limits": K <= 2^17 is the INT8
  accumulator bound.
* enclosure-gemm, "Method": operands are two's-complement integers of up to
  four int64 limbs; one INT8 GEMM per prime below 256; balanced-Garner
  mixed-radix digits in signed 384-bit arithmetic.
* enclosure-gemm, "Requirements and limits": the product of the primes below
  256 is a 335-bit number, and the capacity budget follows from it.
* Ozaki Scheme II paper, §3.1: integer products are exact and there is one
  reconstruction at the end; §1.1: O(p) products, O(p^2) reduction and CRT;
  §3.5.2: the GPU reconstruction takes the centered representative by
  rounding to nearest.

Readings taken where the pages are silent:
  * the prime set for a bound is the *fewest* primes taken largest first;
  * "exceeds" is strict: P > 2 * K * 2^(a_bits + b_bits);
  * a balanced residue of x mod q lies in [-floor((q-1)/2), floor(q/2)]
    (so mod 2 it is 0 or 1);
  * the reconstructed value is the representative in (-P/2, P/2];
  * limbs are little-endian two's complement: lower limbs unsigned, the top
    limb signed, element-major and limb-minor.
"""
from __future__ import annotations

import math
from typing import Iterable, List, Sequence

import numpy as np

# exact-solve, "Requirements and limits": n <= 2^17 (the INT8 accumulator bound).
K_MAX = 1 << 17


# ---------------------------------------------------------------------------
# primes below 256 (exact-solve, "Method"; enclosure-gemm, "Method")
# ---------------------------------------------------------------------------
def primes_below(bound: int = 256) -> List[int]:
    """All primes p < bound, ascending, by trial division."""
    out = []
    for p in range(2, bound):
        if all(p % d for d in range(2, int(math.isqrt(p)) + 1)):
            out.append(p)
    return out


def primes_largest_first(bound: int = 256) -> List[int]:
    """The primes below ``bound``, largest first (251, 241, 239, ...)."""
    return sorted(primes_below(bound), reverse=True)


def prime_power_moduli(bound: int = 256) -> List[int]:
    """For every prime p < bound, the largest power of p not above ``bound``;
    largest first (256, 251, 243, 241, ...).  Their product is lcm(1..256),
    whose log2 is the 362.8-bit INT8 CRT capacity of the Ozaki Scheme II
    paper (§1.2, §4.2.2)."""
    out = []
    for p in primes_below(bound):
        q = p
        while q * p <= bound:
            q *= p
        out.append(q)
    return sorted(out, reverse=True)


def prod(xs: Iterable[int]) -> int:
    r = 1
    for x in xs:
        r *= x
    return r


def prime_set_for_bound(K: int, a_bits: int, b_bits: int) -> List[int]:
    """Fewest largest-first primes below 256 whose product exceeds 2*K*2^(a+b).

    |A| <= 2^a_bits and |B| <= 2^b_bits give |C| <= K * 2^(a_bits+b_bits); the
    representative range of the reconstruction must hold +-that bound
    (exact-solve, "Method": the precision must exceed twice the bound).
    Raises ValueError when even all 54 primes are not enough, or K is outside
    0..2^17.
    """
    if not (0 <= K <= K_MAX):
        raise ValueError("K outside 0..2^17")
    bound2 = 2 * max(K, 1) * (1 << (a_bits + b_bits))
    ps: List[int] = []
    P = 1
    for q in primes_largest_first():
        ps.append(q)
        P *= q
        if P > bound2:
            return ps
    raise ValueError("bound exceeds the product of all primes below 256")


def moduli_set_for_bound(K: int, a_bits: int, b_bits: int, prime_powers: bool = False) -> List[int]:
    """``prime_set_for_bound``, or with ``prime_powers`` the same rule over the
    prime-power moduli (256 first).  Balanced residues mod 256 reach -128, so
    int32 accumulation of K products of them is exact only for K <= 2^17 - 1
    (K * 2^14 <= 2^31 - 1)."""
    if not prime_powers:
        return prime_set_for_bound(K, a_bits, b_bits)
    if not (0 <= K <= K_MAX - 1):
        raise ValueError("K outside 0..2^17-1")
    bound2 = 2 * max(K, 1) * (1 << (a_bits + b_bits))
    ms: List[int] = []
    P = 1
    for q in prime_power_moduli():
        ms.append(q)
        P *= q
        if P > bound2:
            return ms
    raise ValueError("bound exceeds the product of the prime-power moduli")


def limbs_to_hold(P: int) -> int:
    """64-bit limbs needed for every value of (-P/2, P/2] in two's complement.

    A w-bit two's-complement word holds [-2^(w-1), 2^(w-1) - 1]; every value
    of (-P/2, P/2] fits exactly when P < 2^w.
    """
    w = P.bit_length()
    return (w + 63) // 64


# ---------------------------------------------------------------------------
# two's-complement limbs (enclosure-gemm, "Method": up to four int64 limbs)
# ---------------------------------------------------------------------------
_M64 = (1 << 64) - 1


def to_limbs(x: int, L: int) -> List[int]:
    """x -> L int64 limbs, little-endian two's complement.  Raises if x does not fit."""
    if not (-(1 << (64 * L - 1)) <= x < (1 << (64 * L - 1))):
        raise OverflowError(f"{x} does not fit {L} limbs")
    out = []
    for i in range(L):
        u = (x >> (64 * i)) & _M64
        out.append(u - (1 << 64) if u >= (1 << 63) else u)
    return out


def from_limbs(limbs: Sequence[int]) -> int:
    """Inverse of ``to_limbs``: lower limbs read unsigned, the top limb signed."""
    L = len(limbs)
    x = 0
    for i in range(L - 1):
        x += (int(limbs[i]) & _M64) << (64 * i)
    x += int(limbs[L - 1]) << (64 * (L - 1))
    return x


def decode_array(arr: np.ndarray) -> np.ndarray:
    """int64 array [..., L] of limbs -> object array [...] of Python ints."""
    arr = np.asarray(arr)
    assert arr.dtype == np.int64
    L = arr.shape[-1]
    out = arr[..., L - 1].astype(object) * (1 << (64 * (L - 1)))
    for i in range(L - 1):
        out = out + (arr[..., i].view(np.uint64).astype(object) << (64 * i))
    return out


def encode_array(vals: np.ndarray, L: int) -> np.ndarray:
    """object array [...] of Python ints -> int64 array [..., L] (two's complement)."""
    vals = np.asarray(vals, dtype=object)
    out = np.empty(vals.shape + (L,), dtype=np.int64)
    flat = vals.reshape(-1)
    of = out.reshape(-1, L)
    for e, x in enumerate(flat):
        of[e, :] = to_limbs(int(x), L)
    return out


# ---------------------------------------------------------------------------
# balanced residues (exact-solve, "Method"; enclosure-gemm, "Method")
# ---------------------------------------------------------------------------
def balanced(x: int, q: int) -> int:
    """The representative of x mod q in [-floor((q-1)/2), floor(q/2)]."""
    r = x % q                       # Python: 0 <= r < q
    return r - q if r > q // 2 else r


def balanced_array(x: np.ndarray, q: int) -> np.ndarray:
    """Elementwise ``balanced`` on an object or integer array; returns int64."""
    r = np.mod(np.asarray(x, dtype=object), q)
    r = np.where(r > q // 2, r - q, r)
    return r.astype(np.int64)


# ---------------------------------------------------------------------------
# reconstruction (exact-solve, "Method"; Ozaki Scheme II paper §3.1)
# ---------------------------------------------------------------------------
def crt_balanced(residues: Sequence[int], primes: Sequence[int]) -> int:
    """Textbook CRT: the unique X in (-P/2, P/2] with X = r_j (mod q_j) for all j.

    X0 = sum_j r_j * M_j * (M_j^-1 mod q_j) mod P with M_j = P / q_j, then
    the representative is moved into (-P/2, P/2].
    """
    P = prod(primes)
    X0 = 0
    for r, q in zip(residues, primes):
        Mj = P // q
        X0 += int(r) * Mj * pow(Mj, -1, q)
    X0 %= P
    return X0 - P if 2 * X0 > P else X0


def crt_balanced_array(res: Sequence[np.ndarray], primes: Sequence[int]) -> np.ndarray:
    """``crt_balanced`` elementwise over arrays res[j] of residues mod primes[j]."""
    P = prod(primes)
    X0 = np.zeros(np.asarray(res[0]).shape, dtype=object)
    for r, q in zip(res, primes):
        Mj = P // q
        X0 = X0 + np.asarray(r).astype(object) * (Mj * pow(Mj, -1, q))
    X0 = np.mod(X0, P)
    return np.where(2 * X0 > P, X0 - P, X0)


def garner_digits(residues: Sequence[int], primes: Sequence[int]) -> List[int]:
    """Balanced mixed-radix digits d_i with X = sum_i d_i * prod_{k<i} q_k.

    Textbook recurrence: d_i = (r_i - sum_{k<i} d_k prod_{j<k} q_j)
    * (prod_{j<i} q_j)^-1 mod q_i, each digit balanced (exact-solve,
    "Method": balanced Garner).
    """
    ds: List[int] = []
    for i, (r, q) in enumerate(zip(residues, primes)):
        s = 0
        Qk = 1
        for k in range(i):
            s += ds[k] * Qk
            Qk *= primes[k]
        # here Qk = prod_{j<i} q_j
        ds.append(balanced((int(r) - s) * pow(Qk % q, -1, q), q))
    return ds


def mixed_radix_value(digits: Sequence[int], primes: Sequence[int]) -> int:
    X, Q = 0, 1
    for d, q in zip(digits, primes):
        X += d * Q
        Q *= q
    return X


def crt_rounded_quotient(residues: Sequence[int], primes: Sequence[int],
                         quotient_estimate=None) -> int:
    """CRT whose centered representative comes from a rounded quotient.

    Ozaki Scheme II paper, §3.5.2: the GPU reconstruction obtains the
    centered representative by rounding to nearest.  Read plainly:
    u_j = r_j * (M_j^-1 mod q_j) mod q_j (balanced), S = sum_j u_j * M_j with
    M_j = P / q_j, so S = X (mod P) and S / P = sum_j u_j / q_j; the quotient
    t = round(S / P) gives X = S - t * P.

    ``quotient_estimate(u, primes)`` returns the integer t used; by default
    the nearest integer to the exact rational sum_j u_j / q_j.  An estimate
    off by one (a rounded floating-point sum near a half-integer) leaves
    S - t * P one period outside (-P/2, P/2]; one exact comparison with P/2
    moves it back, so the result is the balanced CRT value for any estimate
    within one of the true quotient.
    """
    P = prod(primes)
    u = [balanced(int(r) * pow(P // q, -1, q), q) for r, q in zip(residues, primes)]
    if quotient_estimate is None:
        num = sum(uj * (P // q) for uj, q in zip(u, primes))   # = S; S / P is the sum
        t = (2 * num + P) // (2 * P)                            # nearest, ties upward
    else:
        t = int(quotient_estimate(u, primes))
    X = sum(uj * (P // q) for uj, q in zip(u, primes)) - t * P
    if 2 * X > P:
        X -= P
    elif 2 * X <= -P:
        X += P
    return X


# ---------------------------------------------------------------------------
# the product itself (the definition the method reaches exactly)
# ---------------------------------------------------------------------------
def int_matmul(A: Sequence[Sequence[int]], B: Sequence[Sequence[int]]) -> List[List[int]]:
    """C[i][j] = sum_k A[i][k] * B[k][j] over the integers, by triple loop."""
    M, K = len(A), len(A[0]) if len(A) else 0
    N = len(B[0]) if len(B) else 0
    assert all(len(r) == K for r in A) and len(B) == K
    C = [[0] * N for _ in range(M)]
    for i in range(M):
        Ai = A[i]
        Ci = C[i]
        for j in range(N):
            s = 0
            for k in range(K):
                s += int(Ai[k]) * int(B[k][j])
            Ci[j] = s
    return C


def freivalds_holds(A: np.ndarray, B: np.ndarray, C: np.ndarray, v: np.ndarray) -> bool:
    """Exact check (A @ B) @ v == C @ v ... evaluated as A @ (B @ v) == C @ v.

    A, B, C are object arrays of Python ints, v an integer vector.  A wrong C
    passes one random v in [-2^16, 2^16]^N with probability <= 1/(2^17 + 1).
    """
    v = np.asarray(v).astype(object)
    return bool(np.all(A.dot(B.dot(v)) == C.dot(v)))


# ---------------------------------------------------------------------------
# stage definitions of the residue method (for per-kernel checks)
# ---------------------------------------------------------------------------
def residue_planes(X: np.ndarray, primes: Sequence[int]) -> np.ndarray:
    """int8 planes [n][...]: balanced residue of every entry mod every prime."""
    X = np.asarray(X, dtype=object)
    return np.stack([balanced_array(X, q).astype(np.int8) for q in primes])


def residue_product(Aq: np.ndarray, Bq: np.ndarray, q: int) -> np.ndarray:
    """Balanced ((Aq @ Bq) mod q) for one prime; exact in int64 for K <= 2^17."""
    Y = Aq.astype(np.int64) @ Bq.astype(np.int64)
    return balanced_array(Y, q).astype(np.int8)


def residue_gemm_via_crt(Ares: np.ndarray, B_vals: np.ndarray, primes: Sequence[int]) -> np.ndarray:
    """The batched-residue step, following the method's own steps.

    Ares[j] is an int8 matrix read mod primes[j] (exact-solve, "Method": the
    per-prime inverse applied to the residual is one INT8 GEMM per prime);
    B_vals an object or int64 matrix of integers.  Step 1: r_j = B mod q_j;
    step 2: y_j = (Ares[j] @ r_j) mod q_j; step 3: textbook CRT to the
    representative in (-P/2, P/2].
    """
    res = []
    for j, q in enumerate(primes):
        rq = np.mod(np.asarray(B_vals, dtype=object), q).astype(np.int64)
        yq = np.mod(Ares[j].astype(np.int64) @ rq, q)
        res.append(yq)
    return crt_balanced_array(res, primes)
