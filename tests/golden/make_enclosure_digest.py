"""Write tests/golden/enclosure_digest.json: the SHA-256 of the oracle's
enclosure (lo, hi) of the full-size binary64 product A[1024,4096] @
B[4096,1024] (N(0,1) entries, seed 10), computed by the oracle alone.

    python tests/golden/make_enclosure_digest.py

Route (enclosure-gemm, "Method"): each operand is scaled losslessly by its
coarsest power of two (oracle.enclose.coarsest_lossless_scale), the scaled
integers are laid out as int64 limbs (oracle.oracle.encode_array), their
exact product is formed by the C schoolbook oracle, and every entry of
S * 2^-(Fa+Fb) is rounded outward once with the oracle's Fraction-based
rounding (oracle.enclose.enclose_from_integer), on a pool of host processes.
The digests cover the raw bytes of lo and hi (binary64, row-major)
(enclosure-gemm, "Correctness": SHA-256 over the raw bits).
"""
from __future__ import annotations

import hashlib
import json
import multiprocessing as mp
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)

from oracle import cgemm  # noqa: E402
from oracle import enclose as E  # noqa: E402
from oracle import oracle as O  # noqa: E402
import workloads as W  # noqa: E402

OUT = os.path.join(os.path.dirname(os.path.abspath(__file__)), "enclosure_digest.json")
SEED, M, K, N = 10, 1024, 4096, 1024


def _scaled(args):
    X, F = args
    return E.scaled_integers(X, F)


def _round(args):
    S, Q = args
    return E.enclose_from_integer(S, Q)


def bits_needed(vals) -> int:
    return max(abs(int(v)).bit_length() for v in vals.ravel()) + 1


def main() -> None:
    t0 = time.perf_counter()
    A, B = W.fp64_normal_pair(SEED, M, K, N)
    Fa, Fb = E.coarsest_lossless_scale(A), E.coarsest_lossless_scale(B)
    procs = max(1, len(os.sched_getaffinity(0)))
    with mp.get_context("spawn").Pool(procs) as pool:
        Ai = np.concatenate(pool.map(_scaled, [(c, Fa) for c in np.array_split(A, procs * 4)]))
        Bi = np.concatenate(pool.map(_scaled, [(c, Fb) for c in np.array_split(B, procs * 4)]))
        la = (bits_needed(Ai) + 63) // 64
        lb = (bits_needed(Bi) + 63) // 64
        S = cgemm.gemm(O.encode_array(Ai, la), O.encode_array(Bi, lb), la + lb + 1)
        Sv = O.decode_array(S)
        parts = pool.map(_round, [(c, Fa + Fb) for c in np.array_split(Sv, procs * 4)])
    lo = np.concatenate([p[0] for p in parts])
    hi = np.concatenate([p[1] for p in parts])
    out = {"_about": "SHA-256 of the oracle's outward-rounded enclosure of the full-size binary64 "
                     "product; written by make_enclosure_digest.py from oracle/ only",
           "seed": SEED, "M": M, "K": K, "N": N, "Fa": Fa, "Fb": Fb,
           "inputs_sha256": {"A": hashlib.sha256(A.tobytes()).hexdigest(),
                             "B": hashlib.sha256(B.tobytes()).hexdigest()},
           "lo_sha256": hashlib.sha256(np.ascontiguousarray(lo).tobytes()).hexdigest(),
           "hi_sha256": hashlib.sha256(np.ascontiguousarray(hi).tobytes()).hexdigest()}
    with open(OUT, "w") as f:
        json.dump(out, f, indent=1)
        f.write("\n")
    print(f"Fa={Fa} Fb={Fb} limbs={la},{lb} lo {out['lo_sha256'][:16]} hi {out['hi_sha256'][:16]} "
          f"({time.perf_counter() - t0:.0f} s)", flush=True)


if __name__ == "__main__":
    main()
