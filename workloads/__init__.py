"""Seeded synthetic inputs shared by the tests, the benchmark and the oracle.

This module only draws random numbers (numpy PCG64, one seed per workload) and
lays them out in the operand format: int64 limbs, element-major, limb-minor,
little-endian two's complement.  It holds none of the residue method's
arithmetic; where a workload needs the prime list (the batched-residue step),
the caller passes it in.

The five workloads follow the shapes and value distributions of the pages'
use cases (exact-solve's lift step and enclosure-gemm's fixed-point operands)
at the sizes the benchmark is quoted on:

  tiny       A[64,64] @ B[64,64], entries uniform in [-2^20, 2^20]
  square     A[1024,1024] @ B[1024,1024], entries uniform in [-2^31, 2^31)
  enclosure  A[1024,4096] @ B[4096,1024], floor(N(0,1) * 2^52) (exact in fp64)
  dixon      54 int8 planes [1024,1024] of balanced residues, one per prime,
             times r[1024,16] uniform in [-2^34, 2^34]
  wide       A[2048,4096] @ B[4096,2048], 2-limb entries uniform in [-2^100, 2^100)
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import Dict, List, Optional, Sequence

import numpy as np


@dataclass
class Workload:
    name: str
    M: int
    N: int
    K: int
    A: Optional[np.ndarray]          # int64 [M,K,la]  (None for the batched-residue step)
    B: np.ndarray                    # int64 [K,N,lb]
    a_bits: int                      # declared |A| <= 2^a_bits (-1: residue planes)
    b_bits: int
    A_res: Optional[np.ndarray] = None   # int8 [n,M,K] for the batched-residue step
    n_primes: Optional[int] = None       # fixed prime count (batched-residue step)
    seed: int = 0
    note: str = ""
    extra: Dict = field(default_factory=dict)

    @property
    def la(self) -> int:
        return 0 if self.A is None else self.A.shape[-1]

    @property
    def lb(self) -> int:
        return self.B.shape[-1]


NAMES = ["tiny", "square", "enclosure", "dixon", "wide"]


def _one_limb(x: np.ndarray) -> np.ndarray:
    return np.ascontiguousarray(x.astype(np.int64)[..., None])


def uniform_int64(rng, shape, lo: int, hi: int, endpoint: bool) -> np.ndarray:
    return _one_limb(rng.integers(lo, hi, size=shape, dtype=np.int64, endpoint=endpoint))


def uniform_two_limb(rng, shape, bits: int) -> np.ndarray:
    """Entries uniform in [-2^bits, 2^bits) for 64 < bits < 127, as 2 limbs.

    The low limb is 64 uniform bits; the high limb is uniform in
    [-2^(bits-64), 2^(bits-64)), so hi * 2^64 + lo is uniform on the interval.
    """
    assert 64 < bits < 127
    lo = rng.integers(0, 1 << 64, size=shape, dtype=np.uint64).view(np.int64)
    hi = rng.integers(-(1 << (bits - 64)), 1 << (bits - 64), size=shape, dtype=np.int64)
    return np.ascontiguousarray(np.stack([lo, hi], axis=-1))


def balanced_residue_planes(rng, primes: Sequence[int], M: int, K: int) -> np.ndarray:
    """int8 [n,M,K]: plane j uniform over the balanced residues of primes[j].

    For odd q the values are [-(q-1)/2, (q-1)/2]; for q = 2 they are {0, 1}.
    """
    out = np.empty((len(primes), M, K), dtype=np.int8)
    for j, q in enumerate(primes):
        lo = -((q - 1) // 2)
        hi = q // 2
        out[j] = rng.integers(lo, hi, size=(M, K), dtype=np.int64, endpoint=True).astype(np.int8)
    return out


def bits_bound(x: np.ndarray) -> int:
    """Smallest a with |x| < 2^a for a one-limb array (the declared bound)."""
    m = int(np.max(np.abs(x.astype(np.int64)))) if x.size else 0
    return m.bit_length()


def make(name: str, primes: Optional[Sequence[int]] = None, scale: float = 1.0) -> Workload:
    """Build one named workload.  ``primes`` (largest first) is needed for 'dixon'.

    ``scale`` < 1 shrinks M and N (not K, the distributions or the seed) for
    quick runs; the benchmark and the full-size tests use scale 1.
    """
    def sz(v: int) -> int:
        return max(1, int(round(v * scale)))

    if name == "tiny":
        rng = np.random.default_rng(1)
        M = N = K = 64
        A = uniform_int64(rng, (M, K), -(1 << 20), 1 << 20, endpoint=True)
        B = uniform_int64(rng, (K, N), -(1 << 20), 1 << 20, endpoint=True)
        return Workload(name, M, N, K, A, B, 20, 20, seed=1,
                        note="A[64,64]@B[64,64], uniform [-2^20,2^20]")
    if name == "square":
        rng = np.random.default_rng(2)
        M, N, K = sz(1024), sz(1024), 1024
        A = uniform_int64(rng, (M, K), -(1 << 31), 1 << 31, endpoint=False)
        B = uniform_int64(rng, (K, N), -(1 << 31), 1 << 31, endpoint=False)
        return Workload(name, M, N, K, A, B, 31, 31, seed=2,
                        note="A[1024,1024]@B[1024,1024], uniform [-2^31,2^31)")
    if name == "enclosure":
        rng = np.random.default_rng(3)
        M, N, K = sz(1024), sz(1024), 4096
        # floor(x * 2^52) of an fp64 normal sample is exact: the scaling moves
        # only the exponent and floor() of a double is exact.
        A = _one_limb(np.floor(rng.standard_normal((M, K)) * 2.0 ** 52))
        B = _one_limb(np.floor(rng.standard_normal((K, N)) * 2.0 ** 52))
        return Workload(name, M, N, K, A, B, bits_bound(A), bits_bound(B), seed=3,
                        note="A[1024,4096]@B[4096,1024], floor(N(0,1)*2^52)")
    if name == "dixon":
        if primes is None:
            raise ValueError("the dixon workload needs the prime list")
        rng = np.random.default_rng(4)
        n_sz, c = sz(1024), 16
        r = uniform_int64(rng, (n_sz, c), -(1 << 34), 1 << 34, endpoint=True)
        A_res = balanced_residue_planes(rng, primes, n_sz, n_sz)
        return Workload(name, n_sz, c, n_sz, None, r, -1, 34, A_res=A_res,
                        n_primes=len(primes), seed=4,
                        note="54 x int8 Binv[1024,1024] (balanced mod q_j) @ r[1024,16] uniform [-2^34,2^34]")
    if name == "wide":
        rng = np.random.default_rng(5)
        M, N, K = sz(2048), sz(2048), 4096
        A = uniform_two_limb(rng, (M, K), 100)
        B = uniform_two_limb(rng, (K, N), 100)
        return Workload(name, M, N, K, A, B, 100, 100, seed=5,
                        note="A[2048,4096]@B[4096,2048], 2-limb uniform [-2^100,2^100)")
    raise KeyError(name)


def fp64_normal_pair(seed: int, M: int, K: int, N: int):
    """Binary64 operands A[M,K], B[K,N] with N(0,1) entries (the enclosure
    product's inputs), drawn A first, then B."""
    rng = np.random.default_rng(seed)
    A = rng.standard_normal((M, K))
    B = rng.standard_normal((K, N))
    return A, B


def random_operands(seed: int, M: int, N: int, K: int, la: int, lb: int,
                    a_bits: int, b_bits: int):
    """Generic seeded operands: entries uniform in [-2^bits, 2^bits] as limbs.

    Used for ragged shapes and edge cases.  bits may be up to 64*limbs - 2.
    """
    rng = np.random.default_rng(seed)

    def draw(rows, cols, limbs, bits):
        out = np.zeros((rows, cols, limbs), dtype=np.int64)
        if bits < 63:
            out[..., 0] = rng.integers(-(1 << bits), 1 << bits, size=(rows, cols),
                                       dtype=np.int64, endpoint=True)
            if limbs > 1:
                out[..., 1:] = np.where(out[..., :1] < 0, -1, 0)
            return out
        # multi-limb: random 64-bit lower limbs, signed top part
        full = bits // 64
        for l in range(limbs):
            if l < full:
                out[..., l] = rng.integers(0, 1 << 64, size=(rows, cols), dtype=np.uint64).view(np.int64)
            elif l == full:
                top = bits - 64 * full
                out[..., l] = rng.integers(-(1 << top), 1 << top, size=(rows, cols), dtype=np.int64)
            else:
                out[..., l] = np.where(out[..., full] < 0, -1, 0)
        return out

    return draw(M, K, la, a_bits), draw(K, N, lb, b_bits)
