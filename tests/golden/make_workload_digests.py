"""Write tests/golden/workload_digests.json: SHA-256 digests of the five seeded
workloads' inputs and of their exact products, computed by the oracle alone.

    python tests/golden/make_workload_digests.py

The products come from ``oracle/`` only: the C schoolbook multi-limb product
for the four integer products (the plain definition C = A @ B, which the
residue method reaches exactly), and the method's own steps with the
textbook CRT (``oracle.residue_gemm_via_crt``) for the batched-residue step.
The output width is the oracle's ``limbs_to_hold`` of the product of the
moduli the oracle's prime rule picks.  Digests cover the raw bytes of the
little-endian int64 arrays ([M][N][limbs], limbs innermost), so a GPU result
with the same digest is the same array bit for bit (enclosure-gemm,
"Correctness": SHA-256 over the raw bits).
"""
from __future__ import annotations

import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)

from oracle import cgemm  # noqa: E402
from oracle import oracle as O  # noqa: E402
import workloads as W  # noqa: E402

OUT = os.path.join(os.path.dirname(os.path.abspath(__file__)), "workload_digests.json")


def sha(a: np.ndarray) -> str:
    return hashlib.sha256(np.ascontiguousarray(a).tobytes()).hexdigest()


def main() -> None:
    out = {"_about": "SHA-256 of the seeded workloads' inputs and of their exact products "
                     "(int64 little-endian, [M][N][limbs]); written by make_workload_digests.py "
                     "from oracle/ only"}
    for name in W.NAMES:
        t = time.perf_counter()
        if name == "dixon":
            primes = O.primes_largest_first()
            wl = W.make(name, primes=primes)
            P = O.prod(primes)
            L = O.limbs_to_hold(P)
            X = O.residue_gemm_via_crt(wl.A_res, wl.B[..., 0], primes)
            C = O.encode_array(X, L)
            inputs = {"A_res": sha(wl.A_res), "B": sha(wl.B)}
            n = len(primes)
        else:
            wl = W.make(name)
            primes = O.prime_set_for_bound(wl.K, wl.a_bits, wl.b_bits)
            L = O.limbs_to_hold(O.prod(primes))
            C = cgemm.gemm(wl.A, wl.B, L)
            inputs = {"A": sha(wl.A), "B": sha(wl.B)}
            n = len(primes)
        out[name] = {"M": wl.M, "N": wl.N, "K": wl.K, "n_primes": n, "out_limbs": L,
                     "inputs_sha256": inputs, "C_sha256": sha(C)}
        print(f"{name}: {wl.M}x{wl.N}x{wl.K}, {n} primes, {L} limbs, "
              f"{time.perf_counter() - t:.1f} s, C {out[name]['C_sha256'][:16]}", flush=True)
    with open(OUT, "w") as f:
        json.dump(out, f, indent=1)
        f.write("\n")


if __name__ == "__main__":
    main()
