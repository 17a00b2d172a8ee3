"""Exact rational solve A x = b by Dixon p-adic lifting (C ABI: ``include/rns_solve.h``).

``X = solve(A, b)`` returns the exact solution as lists of ``fractions.Fraction``
(None if A is singular), following exact-solve, "Method": the batched modular
inverse (Gauss-Jordan mod every odd prime below 256 at once) and the lift (one
batched INT8 product per prime per step, the wide digit by the CRT, the
residual in one limb) run in the library's HIP kernels; the rational
reconstruction of x mod P^m runs on the host, as the page's CPU stage does.
"""
from __future__ import annotations

import ctypes
import math
from fractions import Fraction
from typing import List, Optional, Sequence

import numpy as np
import torch

from . import Plan, RnsError, _check, _Plan, _stream_ptr, load

# the odd primes below 256, largest first (P must be odd for the residual update)
ODD_PRIMES = [q for q in range(255, 2, -1) if q % 2 and all(q % d for d in range(3, int(q ** 0.5) + 1, 2))]


def _i32_array(vals: Sequence[int]):
    arr = (ctypes.c_int32 * len(vals))(*[int(v) for v in vals])
    return arr


def _need_int64(t: torch.Tensor, ndim: int, name: str) -> None:
    if not isinstance(t, torch.Tensor) or t.device.type != "cuda" or t.dtype != torch.int64:
        raise ValueError(f"{name} must be an int64 tensor on a GPU device")
    if t.dim() != ndim or not t.is_contiguous():
        raise ValueError(f"{name} must be a contiguous {ndim}-d tensor")


def plan_from_moduli(moduli: Sequence[int], k_max: int) -> Plan:
    c = _Plan()
    _check(load().rns_plan_from_moduli(_i32_array(moduli), len(moduli), k_max, ctypes.byref(c)),
           "rns_plan_from_moduli")
    return Plan._from_c(c)


def batched_inverse(A: torch.Tensor, primes: Sequence[int] = ODD_PRIMES):
    """Gauss-Jordan inverses of A mod every prime.  Returns (singular flags
    (int32 [E] on the device), workspace holding the inverses)."""
    _need_int64(A, 2, "A")
    n = A.shape[0]
    if A.shape[1] != n:
        raise ValueError("A must be square")
    sz = ctypes.c_size_t()
    _check(load().rns_inverse_workspace_size(len(primes), n, ctypes.byref(sz)), "rns_inverse_workspace_size")
    ws = torch.empty(sz.value, dtype=torch.uint8, device=A.device)
    singular = torch.empty(len(primes), dtype=torch.int32, device=A.device)
    with torch.cuda.device(A.device):
        rc = load().rns_batched_inverse(_i32_array(primes), len(primes), n, A.data_ptr(), singular.data_ptr(),
                                        ws.data_ptr(), ws.numel(), _stream_ptr(A))
    _check(rc, "rns_batched_inverse")
    return singular, ws


def inverse_planes(ws: torch.Tensor, n: int, select: Sequence[int], primes: Sequence[int] = ODD_PRIMES):
    """Balanced int8 planes [len(select), n, n] of the inverses mod primes[select]."""
    planes = torch.empty((len(select), n, n), dtype=torch.int8, device=ws.device)
    with torch.cuda.device(ws.device):
        rc = load().rns_inverse_planes(_i32_array(primes), len(primes), n, _i32_array(select), len(select),
                                       planes.data_ptr(), ws.data_ptr(), ws.numel(),
                                       torch.cuda.current_stream(ws.device).cuda_stream)
    _check(rc, "rns_inverse_planes")
    return planes


def dixon_lift(p: Plan, A: torch.Tensor, b: torch.Tensor, planes: torch.Tensor, steps: int) -> torch.Tensor:
    """Digits int64 [steps, n, c, out_limbs_min]: x_i = B r_i mod P, balanced."""
    _need_int64(A, 2, "A")
    _need_int64(b, 2, "b")
    n, c = b.shape
    c_plan = p._c()
    sz = ctypes.c_size_t()
    _check(load().rns_lift_workspace_size(ctypes.byref(c_plan), n, c, ctypes.byref(sz)), "rns_lift_workspace_size")
    ws = torch.empty(sz.value, dtype=torch.uint8, device=A.device)
    dl = p.out_limbs_min
    digits = torch.empty((steps, n, c, dl), dtype=torch.int64, device=A.device)
    with torch.cuda.device(A.device):
        rc = load().rns_dixon_lift(ctypes.byref(c_plan), n, c, planes.data_ptr(), A.data_ptr(), b.data_ptr(), steps,
                                   digits.data_ptr(), dl, ws.data_ptr(), ws.numel(), _stream_ptr(A))
    _check(rc, "rns_dixon_lift")
    return digits


# ---- host stage: bounds and rational reconstruction --------------------------------
def _ceil_sqrt(v: int) -> int:
    r = math.isqrt(v)
    return r if r * r == v else r + 1


def _bounds(A: np.ndarray, b: np.ndarray):
    """Hadamard: |det A| <= prod of row norms; a Cramer numerator replaces a
    column by one of b, so each of its rows is bounded by sqrt(|a_i|^2 + b_ik^2)."""
    n = A.shape[0]
    big = max([max(int(x.max()), -int(x.min())) for x in (A, b) if x.size] or [0])
    if (n + 1) * big * big < 1 << 63:           # the squared norms are exact in int64
        A64 = A.astype(np.int64, copy=False)
        b64 = b.astype(np.int64, copy=False)
        rows2 = np.einsum("ij,ij->i", A64, A64).tolist()
        b2 = (b64 * b64).tolist()
    else:
        rows2 = [sum(int(v) * int(v) for v in row) for row in A.tolist()]
        b2 = [[int(v) * int(v) for v in row] for row in b.tolist()]
    D = _prod_tree([_ceil_sqrt(r2) for r2 in rows2])
    N = 1
    for k in range(b.shape[1]):
        N = max(N, _prod_tree([_ceil_sqrt(r2 + b2[i][k]) for i, r2 in enumerate(rows2)]))
    return N, max(D, 1)


def _prod_tree(vals: List[int]) -> int:
    """The product of many integers by pairwise rounds (balanced operand sizes)."""
    vals = list(vals) or [1]
    while len(vals) > 1:
        nxt = [vals[i] * vals[i + 1] for i in range(0, len(vals) - 1, 2)]
        if len(vals) % 2:
            nxt.append(vals[-1])
        vals = nxt
    return vals[0]


def _limbs_to_int(limbs: np.ndarray) -> List[int]:
    """int64 [..., L] two's-complement limbs -> Python ints (flattened)."""
    L = limbs.shape[-1]
    flat = np.ascontiguousarray(limbs.reshape(-1, L), dtype=np.int64)
    raw = memoryview(flat).cast("B")          # no copy
    w = 8 * L
    return [int.from_bytes(raw[i * w:(i + 1) * w], "little", signed=True) for i in range(flat.shape[0])]


def _mag(v: int):
    """A non-negative int as little-endian uint64 limbs (at least one)."""
    n = max(1, (v.bit_length() + 63) // 64)
    return np.frombuffer(v.to_bytes(8 * n, "little"), dtype=np.uint64).copy(), n


def _ptr(a: np.ndarray) -> int:
    return a.ctypes.data


def host_bigint_available() -> bool:
    """Whether the native host stage (GMP through the library) can run."""
    return bool(load().rns_host_bigint_available())


def padic_numerators(digits: np.ndarray, P: int, D: int, bound: int, index: Optional[Sequence[int]] = None,
                     threads: int = 0):
    """For the components ``index`` of digits int64 [steps, count, L]: w = D * X mod P^steps (balanced),
    X = sum_s digits[s] P^s; returns (ok bool [len(index)], w as ints, 0 where not ok)."""
    digits = np.ascontiguousarray(digits, dtype=np.int64)
    steps, count, L = digits.shape
    idx = np.arange(count, dtype=np.int64) if index is None else np.ascontiguousarray(index, dtype=np.int64)
    Pl, pn = _mag(P)
    Dl, dn = _mag(D)
    Bl, bn = _mag(bound)
    wl = bound.bit_length() // 64 + 1
    num = np.zeros((max(len(idx), 1), wl), dtype=np.int64)
    ok = np.zeros(max(len(idx), 1), dtype=np.int32)
    rc = load().rns_padic_numerators(_ptr(digits), steps, count, L, _ptr(idx), len(idx), _ptr(Pl), pn, _ptr(Dl), dn,
                                     _ptr(Bl), bn, _ptr(num), wl, _ptr(ok), threads)
    _check(rc, "rns_padic_numerators")
    return ok[:len(idx)].astype(bool), _limbs_to_int(num[:len(idx)])


def rational_reconstruct(u: int, M: int, Nb: int, Db: int) -> Optional[Fraction]:
    """N/d with |N| <= Nb, 0 < d <= Db, N = d u (mod M) (native extended Euclid); None if none."""
    ul, un = _mag(u if u >= 0 else u % M)       # the native call reduces mod M
    Ml, mn = _mag(M)
    Nl, nn = _mag(Nb)
    Dl, dn = _mag(Db)
    numl = Nb.bit_length() // 64 + 1
    num = np.zeros(numl, dtype=np.int64)
    den = np.zeros(dn, dtype=np.uint64)
    rc = load().rns_rational_reconstruct(_ptr(ul), un, _ptr(Ml), mn, _ptr(Nl), nn, _ptr(Dl), dn, _ptr(num), numl,
                                         _ptr(den), dn)
    if rc == -8:
        return None
    _check(rc, "rns_rational_reconstruct")
    return Fraction(_limbs_to_int(num.reshape(1, -1))[0], int.from_bytes(den.tobytes(), "little"))


def _ratrec(u: int, M: int, Nb: int, Db: int) -> Optional[Fraction]:
    r0, r1, t0, t1 = M, u % M, 0, 1
    while r1 > Nb:
        qt = r0 // r1
        r0, r1 = r1, r0 - qt * r1
        t0, t1 = t1, t0 - qt * t1
    if t1 == 0 or abs(t1) > Db or (r1 - t1 * u) % M:
        return None
    return Fraction(r1, t1)


def lift_steps_for(P: int, Nb: int, Db: int) -> int:
    """The least m with P^m > 2 Nb Db (Db + 1): enough for one rational
    reconstruction per denominator and a rigorous one-multiply test for every
    other component."""
    target = 2 * Nb * Db * (Db + 1)
    # start just below the answer from the bit lengths, then step
    m = max(1, int(target.bit_length() / math.log2(P)) - 1)
    Pm = P ** m
    while Pm > target and m > 1:
        m -= 1
        Pm //= P
    while Pm <= target:
        m += 1
        Pm *= P
    return m


def reconstruct(per_step: Sequence[Sequence[int]], P: int, m: int, Nb: int, Db: int):
    """(numerators, common denominator) from the lift digits per_step[s][idx].

    x = sum_s digits[s] P^s mod P^m per component.  Common denominator D:
    w = D u mod P^m (balanced) is the numerator over D when |w| <= D Nb --
    rigorous, since a wrong w would give |w e - D a| < P^m for the true a/e,
    so e | D.  Otherwise the component is reconstructed alone (unique for
    P^m > 2 Nb Db) and D grows."""
    Pm = P ** m
    count = len(per_step[0])
    D = 1
    nums: List[int] = []
    half = Pm // 2
    for idx in range(count):
        v = 0
        for s in range(m - 1, -1, -1):
            v = v * P + per_step[s][idx]
        u = v % Pm
        w = D * u % Pm
        if w > half:
            w -= Pm
        if abs(w) > D * Nb:
            f = _ratrec(u, Pm, Nb, Db)
            if f is None:
                raise RnsError(-8, "rational reconstruction failed")
            g = f.denominator // math.gcd(D, f.denominator)
            nums = [x * g for x in nums]
            D *= g
            w = D * u % Pm
            if w > half:
                w -= Pm
        nums.append(w)
    return nums, D


def reconstruct_digits(digits: np.ndarray, P: int, m: int, Nb: int, Db: int, threads: int = 0):
    """(numerators, common denominator) from the lift digits int64 [m, count, L], in native code.

    The first component still pending is reconstructed alone (its p-adic value, then the extended
    Euclidean algorithm); the common denominator D takes its denominator, and one pass over every
    pending component computes w = D u mod P^m and keeps those with |w| <= D Nb (rigorous for
    P^m > 2 Nb Db (Db + 1), as in ``reconstruct``).  Components that fail wait for the next
    denominator; each pass at least doubles D, so there are at most log2 Db + 1 passes."""
    digits = np.ascontiguousarray(digits, dtype=np.int64)
    return _reconstruct_with(lambda D, bound, idx, th: padic_numerators(digits, P, D, bound, idx, th),
                             digits.shape[1], P, m, Nb, Db, threads)


def pow_table(P: int, m: int, T: int) -> np.ndarray:
    """int64 [T][m]: entry [t][s] is 32-bit chunk t of P^s (native when GMP is there)."""
    if host_bigint_available():
        out = np.zeros((T, m), dtype=np.int64)
        Pl, pn = _mag(P)
        _check(load().rns_pow_table(_ptr(Pl), pn, m, T, _ptr(out)), "rns_pow_table")
        return out
    tab = np.zeros((m, T), dtype=np.uint32)
    v = 1
    for s in range(m):
        raw = np.frombuffer(v.to_bytes(4 * T, "little"), dtype=np.uint32)
        tab[s] = raw
        v *= P
    return np.ascontiguousarray(tab.T.astype(np.int64))


def chunk_count(P: int, m: int) -> int:
    """32-bit chunks holding every balanced value mod P^m in two's complement."""
    return ((P ** m).bit_length() + 1 + 31) // 32


def padic_chunks(digits: torch.Tensor, P: int, m: int, table: Optional[np.ndarray] = None,
                 transposed: bool = False) -> torch.Tensor:
    """The p-adic values sum_s digits[s] P^s of every component as 32-bit two's-complement chunks,
    int32 [count, T] on the device (rns_padic_chunks: two exact residue products and a carry pass),
    or with ``transposed`` int64 [T, count] chunk values (the top one signed).
    ``table`` is ``pow_table(P, m, chunk_count(P, m))`` when the caller built it already (say while
    the lift ran)."""
    if digits.dim() != 3 or digits.dtype != torch.int64 or digits.device.type != "cuda":
        raise ValueError("digits must be an int64 [m, count, limbs] tensor on a GPU device")
    digits = digits.contiguous()
    _, count, dl = digits.shape
    T = chunk_count(P, m)
    if table is None:
        table = pow_table(P, m, T)
    if table.shape != (T, m):
        raise ValueError("table must be pow_table(P, m, chunk_count(P, m))")
    pw = torch.from_numpy(np.ascontiguousarray(table, dtype=np.int64)).to(digits.device)
    sz = ctypes.c_size_t()
    _check(load().rns_padic_chunks_workspace_size(T, m, count, dl, P.bit_length(), ctypes.byref(sz)),
           "rns_padic_chunks_workspace_size")
    ws = torch.empty(max(sz.value, 1), dtype=torch.uint8, device=digits.device)
    if transposed:
        out = torch.empty((T, count), dtype=torch.int64, device=digits.device)
    else:
        out = torch.empty((count, T), dtype=torch.int32, device=digits.device)
    with torch.cuda.device(digits.device):
        rc = load().rns_padic_chunks(pw.data_ptr(), T, m, digits.data_ptr(), count, dl, P.bit_length(),
                                     int(transposed), out.data_ptr(), ws.data_ptr(), ws.numel(),
                                     _stream_ptr(digits))
    _check(rc, "rns_padic_chunks")
    return out


def _chunks_of(v: int, n: Optional[int] = None) -> np.ndarray:
    """int64 vector of the 32-bit chunks of a non-negative integer (n of them, or as many as needed)."""
    n = max(1, (v.bit_length() + 31) // 32) if n is None else n
    return np.frombuffer(v.to_bytes(4 * n, "little"), dtype=np.uint32).astype(np.int64)


class ModmulConstants:
    """The fixed part of the GPU's one modular multiply per numerator (``chunk_modmul``) for P^m and
    a denominator bound Db, computable before the digits exist (say while the lift runs).

    With L = bits(P^m) and G = 64 guard bits: s1 = 32 floor((L - 1 - G) / 32), so 2^s1 <= P^m 2^-G;
    |a| = |floor(D X / 2^s1)| <= Db P^m / 2^(s1 + 1) + 1 < 2^abits for any D <= Db and
    |X| <= P^m / 2; k2 = 32 ceil((abits + G) / 32); mu = floor(2^(s1 + k2) / P^m).  Then the
    rounded quotient is within 1/2 + 2^(1 - G) of D X / P^m, and Tw chunks hold |w| < P^m."""

    G = 64

    def __init__(self, P: int, m: int, Db: int, device):
        Pm = P ** m
        L = Pm.bit_length()
        self.s1c = (L - 1 - self.G) // 32
        abits = Db.bit_length() + L - 32 * self.s1c + 1
        self.k2c = (abits + self.G + 31) // 32
        e = 32 * (self.s1c + self.k2c)
        if host_bigint_available():
            Pl, pn = _mag(Pm)
            ql = (e - L + 1) // 64 + 2
            q = np.zeros(ql, dtype=np.uint64)
            _check(load().rns_pow2_quotient(e, _ptr(Pl), pn, _ptr(q), ql), "rns_pow2_quotient")
            mu = int.from_bytes(q.tobytes(), "little")
        else:
            mu = (1 << e) // Pm
        self.Tw = L // 32 + 2
        self.mu = torch.from_numpy(_chunks_of(mu)).to(device)
        self.Pm = torch.from_numpy(_chunks_of(Pm)).to(device)


def chunk_modmul(Xt: torch.Tensor, D: int, consts: ModmulConstants) -> torch.Tensor:
    """w0 = D X - q P^m mod 2^(32 Tw) for every component (uint32 chunks as int32 [count, Tw] on the
    device; rns_chunk_modmul): D X mod P^m up to one correction by +-P^m."""
    if Xt.dim() != 2 or Xt.dtype != torch.int64 or Xt.device.type != "cuda":
        raise ValueError("Xt must be an int64 [T, count] tensor on a GPU device")
    Xt = Xt.contiguous()
    T, count = Xt.shape
    Dc = torch.from_numpy(_chunks_of(D)).to(Xt.device)
    args = (T, count, Dc.numel(), consts.mu.numel(), consts.Pm.numel(), consts.s1c, consts.k2c, consts.Tw)
    sz = ctypes.c_size_t()
    _check(load().rns_chunk_modmul_workspace_size(*args, ctypes.byref(sz)), "rns_chunk_modmul_workspace_size")
    ws = torch.empty(max(sz.value, 1), dtype=torch.uint8, device=Xt.device)
    out = torch.empty((count, consts.Tw), dtype=torch.int32, device=Xt.device)
    with torch.cuda.device(Xt.device):
        rc = load().rns_chunk_modmul(Xt.data_ptr(), T, count, Dc.data_ptr(), Dc.numel(), consts.mu.data_ptr(),
                                     consts.mu.numel(), consts.Pm.data_ptr(), consts.Pm.numel(), consts.s1c,
                                     consts.k2c, consts.Tw, out.data_ptr(), ws.data_ptr(), ws.numel(),
                                     _stream_ptr(Xt))
    _check(rc, "rns_chunk_modmul")
    return out


def chunk_bound(w: torch.Tensor, bound: int):
    """(ok, numerators, used) on the device for chunk values w (int32 [count, Tw]): ok = |w| <=
    bound, the numerator w as int64 limbs [count, limbs] when ok, and the limbs each accepted
    numerator needs with its sign (rns_chunk_bound)."""
    count, Tw = w.shape
    B = torch.from_numpy(_chunks_of(bound).astype(np.uint32).view(np.int32)).to(w.device)
    wl = bound.bit_length() // 64 + 1
    num = torch.empty((max(count, 1), wl), dtype=torch.int64, device=w.device)
    ok = torch.empty(max(count, 1), dtype=torch.int32, device=w.device)
    used = torch.empty(max(count, 1), dtype=torch.int32, device=w.device)
    with torch.cuda.device(w.device):
        rc = load().rns_chunk_bound(w.data_ptr(), Tw, count, B.data_ptr(), B.numel(), num.data_ptr(), wl,
                                    ok.data_ptr(), used.data_ptr(), _stream_ptr(w))
    _check(rc, "rns_chunk_bound")
    return ok[:count], num[:count], used[:count]


def chunk_numerators(chunks: np.ndarray, P: int, m: int, D: int, bound: int, index=None, threads: int = 0):
    """``padic_numerators`` with the p-adic values given as chunks (uint32 [count][T])."""
    chunks = np.ascontiguousarray(chunks).view(np.uint32)
    count, T = chunks.shape
    idx = np.arange(count, dtype=np.int64) if index is None else np.ascontiguousarray(index, dtype=np.int64)
    Pl, pn = _mag(P)
    Dl, dn = _mag(D)
    Bl, bn = _mag(bound)
    wl = bound.bit_length() // 64 + 1
    num = np.zeros((max(len(idx), 1), wl), dtype=np.int64)
    ok = np.zeros(max(len(idx), 1), dtype=np.int32)
    rc = load().rns_chunk_numerators(_ptr(chunks), T, count, _ptr(idx), len(idx), _ptr(Pl), pn, m, _ptr(Dl), dn,
                                     _ptr(Bl), bn, _ptr(num), wl, _ptr(ok), threads)
    _check(rc, "rns_chunk_numerators")
    return ok[:len(idx)].astype(bool), _limbs_to_int(num[:len(idx)])


def _sample_modulus(P: int, Nb: int, Db: int) -> int:
    """The least power P^k > 2 Nb Db: a component reconstructed alone has a unique fraction there."""
    target = 2 * Nb * Db
    k = max(1, int(target.bit_length() / math.log2(P)) - 1)     # just below, from the bit lengths
    Pk = P ** k
    while Pk > target and k > 1:
        k -= 1
        Pk //= P
    while Pk <= target:
        Pk *= P
    return Pk


def _reconstruct_with(numerators, count: int, P: int, m: int, Nb: int, Db: int, threads: int = 0,
                      Pm: Optional[int] = None, Pk: Optional[int] = None):
    """The common-denominator loop of ``reconstruct_digits`` over a numerators source.  A component
    reconstructed alone needs only P^k > 2 Nb Db (its fraction is unique there), so its Euclidean
    remainder sequence runs on u mod P^k; the one-multiply test of the others keeps P^m."""
    Pm = P ** m if Pm is None else Pm
    Pk = _sample_modulus(P, Nb, Db) if Pk is None else Pk
    D = 1
    nums: List[Optional[int]] = [None] * count
    at: List[int] = [1] * count
    todo = np.arange(count, dtype=np.int64)
    while len(todo):
        _, (u,) = numerators(1, Pm // 2, todo[:1], 1)
        # u + P^m is non-negative and congruent to u mod P^k (P^k divides P^m); the native call
        # reduces it
        f = rational_reconstruct(u + Pm if u < 0 else u, Pk, Nb, Db)
        if f is None:
            raise RnsError(-8, "rational reconstruction failed")
        D *= f.denominator // math.gcd(D, f.denominator)
        ok, w = numerators(D, D * Nb, todo, threads)
        if not ok[0]:
            raise RnsError(-8, "a reconstructed component failed the common-denominator test")
        for t in np.flatnonzero(ok):
            nums[todo[t]] = w[t]
            at[todo[t]] = D
        todo = todo[~ok]
    if all(a is D for a in at):        # one denominator for every component: the common case
        return nums, D
    scale = {a: D // a for a in set(at)}
    return [v * scale[a] for v, a in zip(nums, at)], D


def reconstruct_chunks(chunks: np.ndarray, P: int, m: int, Nb: int, Db: int, threads: int = 0):
    """(numerators, common denominator) from the p-adic values as chunks (``padic_chunks``)."""
    chunks = np.ascontiguousarray(chunks).view(np.uint32)
    return _reconstruct_with(lambda D, bound, idx, th: chunk_numerators(chunks, P, m, D, bound, idx, th),
                             chunks.shape[0], P, m, Nb, Db, threads)


class ReconstructionPrep:
    """What the reconstruction needs before the digits exist: the power table of ``padic_chunks``
    and the constants of ``chunk_modmul`` (built on the host while the lift runs)."""

    def __init__(self, P: int, m: int, Db: int, device, Nb: Optional[int] = None, count: int = 0):
        self.table = pow_table(P, m, chunk_count(P, m))
        self.consts = ModmulConstants(P, m, Db, device)
        self.Pm = P ** m
        self.Pk = _sample_modulus(P, Nb, Db) if Nb is not None else None
        # pinned host memory for the numerators (every bound D Nb with D <= Db fits)
        self.pinned = None
        if Nb is not None and count > 0:
            wl = (Db * Nb).bit_length() // 64 + 1
            self.pinned = torch.empty(count * wl, dtype=torch.int64, pin_memory=True)


def reconstruct_device(digits: torch.Tensor, P: int, m: int, Nb: int, Db: int,
                       prep: Optional[ReconstructionPrep] = None):
    """The reconstruction of device digits [m, count, limbs]: the p-adic values in binary and the
    one modular multiply per numerator on the GPU; the sample's rational reconstruction, the
    +-P^m correction and the bound test on the host (native; Python integers without GMP)."""
    if host_bigint_available():
        if prep is None:
            prep = ReconstructionPrep(P, m, Db, digits.device, Nb, digits.shape[1])
        Xt = padic_chunks(digits, P, m, prep.table, transposed=True)
        count = Xt.shape[1]
        cache = {}

        half = P ** m // 2

        def numerators(D, bound, idx, threads):
            if D == 1 and bound >= half:
                # the balanced p-adic values themselves, from their chunk values
                cols = Xt[:, torch.as_tensor(idx, device=Xt.device)].t().cpu().numpy()
                raw = np.ascontiguousarray(cols.astype(np.uint32)).tobytes()
                w = 4 * cols.shape[1]
                return (np.ones(len(idx), dtype=bool),
                        [int.from_bytes(raw[i * w:(i + 1) * w], "little", signed=True) for i in range(len(idx))])
            if D > Db:
                raise RnsError(-8, "a common denominator above the determinant bound")
            key = (D, bound)
            if key not in cache:
                # D x mod P^m and the bound test on the GPU for every component (P^m > 2 D Nb (Db + 1))
                cache.clear()
                ok_d, num_d, used_d = chunk_bound(chunk_modmul(Xt, D, prep.consts), bound)
                # copy only the limbs the widest accepted numerator needs
                u = max(1, int(used_d.max()))                                      # synchronises
                num_d = num_d[:, :u].contiguous()
                if prep.pinned is not None and prep.pinned.numel() >= num_d.numel():
                    num_h = prep.pinned[:num_d.numel()].view(num_d.shape)
                    num_h.copy_(num_d)                                             # synchronises
                else:
                    num_h = num_d.cpu()
                cache[key] = (ok_d.cpu().numpy().astype(bool), num_h.numpy())
            ok_all, num_all = cache[key]
            sel = np.asarray(idx, dtype=np.int64)
            ok = ok_all[sel]
            return ok, _limbs_to_int(num_all[sel])

        return _reconstruct_with(numerators, count, P, m, Nb, Db, Pm=prep.Pm, Pk=prep.Pk)
    d = digits.cpu().numpy()
    per_step = [_limbs_to_int(d[s]) for s in range(m)]
    return reconstruct(per_step, P, m, Nb, Db)


def _make_reduced(frac=Fraction):
    """A constructor of N/D already in lowest terms: Fraction's private
    ``_normalize=False`` skips the gcd where the running Python has it (3.10 and
    3.11); elsewhere the plain constructor (which repeats the gcd, same value)."""
    try:
        frac(1, 1, _normalize=False)
    except TypeError:
        return frac
    return lambda n, d: frac(n, d, _normalize=False)


_reduced_fraction = _make_reduced()


def to_fractions(nums: Sequence[int], D: int, threads: int = 0) -> List[Fraction]:
    """[N_i / D] in lowest terms; the gcds on host threads by GMP when it is there (Python's gcd of
    two 27,000-bit numbers takes about a millisecond, and an n = 1024 solve has 1024 of them)."""
    if not nums:
        return []
    if not host_bigint_available():
        return [Fraction(v, D) for v in nums]
    L = max(abs(v).bit_length() for v in nums) // 64 + 1
    num = np.frombuffer(b"".join(v.to_bytes(8 * L, "little", signed=True) for v in nums),
                        dtype=np.int64).reshape(len(nums), L)
    Dl, dn = _mag(D)
    num_out = np.zeros_like(num)
    den_out = np.zeros((len(nums), dn), dtype=np.uint64)
    _check(load().rns_reduce_fractions(_ptr(num), len(nums), L, _ptr(Dl), dn, _ptr(num_out), _ptr(den_out),
                                       threads), "rns_reduce_fractions")
    red = _limbs_to_int(num_out)
    raw = memoryview(den_out).cast("B")
    w = 8 * dn
    return [_reduced_fraction(v, int.from_bytes(raw[i * w:(i + 1) * w], "little")) for i, v in enumerate(red)]


def solve(A: torch.Tensor, b: torch.Tensor, return_info: bool = False):
    """Exact x with A x = b as [n][c] lists of Fraction; None if A is singular."""
    _need_int64(A, 2, "A")
    if b.dim() == 1:
        b = b.reshape(-1, 1)
    _need_int64(b.contiguous(), 2, "b")
    b = b.contiguous()
    n = A.shape[0]
    if A.shape != (n, n) or b.shape[0] != n:
        raise ValueError("A must be [n, n] and b [n, c]")
    if b.shape[1] == 0:
        raise ValueError("b needs at least one column")
    if n == 0:
        return ([], {"primes": [], "steps": 0, "numerators": [], "denominator": 1}) if return_info else []
    An = A.cpu().numpy()
    bn = b.cpu().numpy()
    amax = max(int(An.max()), -int(An.min())) if n else 0     # exact: Python ints, no int64 overflow
    if n * amax >= 1 << 63:
        raise ValueError("n * max|A| must stay below 2^63 (the residual is one signed limb)")
    singular, ws = batched_inverse(A)
    Nb, Db = _bounds(An, bn)                           # on the host while the inverse runs
    sing = singular.cpu().tolist()                     # synchronises
    sel = [i for i, s in enumerate(sing) if not s]
    if not sel:
        # det A vanishes mod every odd prime below 256, hence mod their product; below that product
        # (Hadamard) it is zero, so A is singular over the rationals.
        if Db < math.prod(ODD_PRIMES):
            return None
        raise RnsError(-3, "A is singular modulo every odd prime below 256, but det A may be nonzero")
    moduli = [ODD_PRIMES[i] for i in sel]
    p = plan_from_moduli(moduli, max(n, 1))
    planes = inverse_planes(ws, n, sel)
    del ws
    P = math.prod(moduli)
    m = lift_steps_for(P, Nb, Db)
    digits = dixon_lift(p, A, b, planes, m)
    # the lift runs asynchronously: build the reconstruction's tables on the host meanwhile
    prep = ReconstructionPrep(P, m, Db, A.device, Nb, n * bn.shape[1]) if host_bigint_available() else None
    c = bn.shape[1]
    nums, D = reconstruct_device(digits.reshape(m, n * c, -1), P, m, Nb, Db, prep)
    fr = to_fractions(nums, D)
    out = [[fr[i * c + k] for k in range(c)] for i in range(n)]
    if return_info:
        return out, {"primes": moduli, "steps": m, "log2_P": math.log2(P), "denominator_bits": D.bit_length(),
                     "numerators": nums, "denominator": D}
    return out
