"""Parity of the HIP path with the CPU oracle, element by element (GPU only).

Every comparison is bit-exact: the path computes integers.  Small and medium
shapes (several tiles plus a ragged tail in M, N and K) are compared in full
against the C oracle; stage-level checks compare the residue planes the split
kernel wrote, and the per-prime products the MFMA kernel wrote, with the
oracle's stage definitions.  The five full-size workloads are compared in
full with the oracle, element by element, and by the SHA-256 of the output
bytes against the digest the oracle alone wrote into
tests/golden/workload_digests.json (enclosure-gemm, "Correctness": SHA-256
over the raw bits).
"""
import hashlib
import json
import os

import numpy as np
import pytest
import torch

import exact_integer_gemm_amd as rg
import workloads as W
from oracle import oracle as O
from oracle import cgemm

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _setup():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    rg.load()
    cgemm.build()
    yield


def dev(x):
    return torch.from_numpy(np.ascontiguousarray(x)).cuda()


def run_gemm(A, B, a_bits, b_bits, out_limbs=None, plan=None):
    K = A.shape[1]
    p = plan or rg.plan(K, a_bits, b_bits)
    ws = rg.new_workspace(p, A.shape[0], B.shape[1], K)
    C = rg.gemm(p, dev(A), dev(B), out_limbs=out_limbs, workspace=ws)
    torch.cuda.synchronize()
    return p, ws, C.cpu().numpy()


def oracle_c(A, B, lc):
    return cgemm.gemm(A, B, lc)


SMALL = [
    # M, N, K, la, lb, a_bits, b_bits, seed
    (64, 64, 64, 1, 1, 20, 20, 11),       # one small tile
    (70, 50, 130, 2, 1, 90, 40, 12),      # ragged everywhere
    (1, 1, 1, 1, 1, 62, 62, 13),          # single entry
    (33, 97, 65, 3, 2, 150, 100, 14),     # wide operands, ragged
    (128, 24, 200, 1, 1, 62, 30, 15),     # skinny N (lift-step tiling)
    (300, 280, 257, 1, 1, 40, 40, 16),    # small tiles, several per prime
    (512, 512, 320, 2, 2, 100, 100, 17),  # big tiles
    (513, 260, 129, 4, 4, 150, 160, 18),  # big tiles + ragged + 4 limbs
    (17, 5, 4096, 1, 2, 60, 90, 19),      # long K, tiny output
]


@pytest.mark.parametrize("M,N,K,la,lb,ab,bb,seed", SMALL)
def test_product_exact_small(M, N, K, la, lb, ab, bb, seed):
    print(f"case M={M} N={N} K={K} la={la} lb={lb} bits={ab},{bb} seed={seed}", flush=True)
    A, B = W.random_operands(seed, M, N, K, la, lb, ab, bb)
    p, ws, C = run_gemm(A, B, ab, bb)
    ref = oracle_c(A, B, p.out_limbs_min)
    assert C.shape == ref.shape
    assert np.array_equal(C, ref)
    assert rg.status(ws) == 0


# The reconstruction's quad form (four entries per lane pair) runs from
# 1024 groups of 128 entries: flat groups when N is a multiple of 4 below
# 1024 columns, 128-column row groups from 1024 columns (a ragged last group
# here); smaller outputs take the byte form.
QUAD = [
    (520, 276, 70, 1, 2, 50, 90, 41),     # flat quads, N % 128 != 0
    (150, 1100, 33, 2, 1, 100, 40, 42),   # row groups of 128 columns, ragged last group
    (260, 512, 64, 1, 1, 62, 62, 43),     # row groups, N a multiple of 128
]


@pytest.mark.parametrize("M,N,K,la,lb,ab,bb,seed", QUAD)
def test_reconstruction_quad_form(M, N, K, la, lb, ab, bb, seed):
    print(f"quad CRT M={M} N={N} K={K}", flush=True)
    A, B = W.random_operands(seed, M, N, K, la, lb, ab, bb)
    p, ws, C = run_gemm(A, B, ab, bb)
    assert np.array_equal(C, oracle_c(A, B, p.out_limbs_min))
    out = torch.empty((M, N, p.out_limbs_min), dtype=torch.int64, device="cuda")
    rg.reconstruct(p, M, N, K, ws, out, method="garner")
    assert np.array_equal(out.cpu().numpy(), C)


@pytest.mark.parametrize("M,N,K,la,lb,ab,bb,seed", [SMALL[1], SMALL[3], SMALL[4], SMALL[7]])
def test_stage_planes(M, N, K, la, lb, ab, bb, seed):
    """Split planes and per-prime products against the oracle's stage definitions."""
    print(f"stages M={M} N={N} K={K}", flush=True)
    A, B = W.random_operands(seed, M, N, K, la, lb, ab, bb)
    p, ws, C = run_gemm(A, B, ab, bb)
    planes = rg.workspace_planes(p, ws, M, N, K)
    Ap = planes["A"].cpu().numpy()
    Bp = planes["B"].cpu().numpy()
    Yp = planes["Y"].cpu().numpy()
    Av, Bv = O.decode_array(A), O.decode_array(B)
    refA = O.residue_planes(Av, p.primes)
    refB = O.residue_planes(Bv.T, p.primes)
    assert np.array_equal(Ap[:, :M, :K], refA)
    assert not Ap[:, M:, :].any() and not Ap[:, :, K:].any()
    assert np.array_equal(Bp[:, :N, :K], refB)
    assert not Bp[:, N:, :].any() and not Bp[:, :, K:].any()
    for j, q in enumerate(p.primes):
        refY = O.residue_product(refA[j], refB[j].T, q)
        assert np.array_equal(Yp[j, :M, :N], refY), f"prime {q}"


def test_split_tail_tiles():
    """Tiles past the last whole round over the compute units run as K parts
    whose residues the last part to finish combines; the result stays exact,
    and the per-tile counters are back at zero for a second product on the
    same workspace (no split in between)."""
    M, N, K = 512, 768, 1024
    p = rg.plan(K, 142, 142)
    tiles = p.n_primes * (M // 256) * (N // 256)
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    print(f"split tail: M={M} N={N} K={K} n={p.n_primes} tiles={tiles} cus={cus}", flush=True)
    if not (tiles > cus and tiles % cus):
        pytest.skip("shape does not leave a partial round on this device")
    A, B = W.random_operands(31, M, N, K, 3, 3, 142, 142)
    ws = rg.new_workspace(p, M, N, K)
    C = rg.gemm(p, dev(A), dev(B), workspace=ws)
    torch.cuda.synchronize()
    ref = oracle_c(A, B, p.out_limbs_min)
    assert np.array_equal(C.cpu().numpy(), ref)
    for _ in range(2):
        rg.residue_products(p, M, N, K, ws)
        out = torch.full_like(C, -1)
        rg.reconstruct(p, M, N, K, ws, out)
        torch.cuda.synchronize()
        assert np.array_equal(out.cpu().numpy(), ref)


# Shapes whose 256 x 256 tiles exceed a whole round over 256 compute units by
# 14, 26 and 94 tiles: the products split those tiles over K into 16, 8 and
# 2 parts, and the combine adds the parts of each tile's row blocks.  Small
# entries keep the product far inside the capacity of the n primes.
SPLIT_PARTS = [
    # M, N, K, n primes, parts expected on 256 compute units, seed
    (256, 1280, 4096, 54, 16, 41),
    (256, 1536, 2048, 47, 8, 42),
    (256, 1792, 1024, 50, 2, 43),
]


@pytest.mark.parametrize("M,N,K,n,parts,seed", SPLIT_PARTS)
def test_split_tail_part_counts(M, N, K, n, parts, seed):
    tiles = n * (M // 256) * (N // 256)
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    print(f"split tail parts: M={M} N={N} K={K} n={n} tiles={tiles} cus={cus} "
          f"(parts {parts} on 256 compute units)", flush=True)
    p = rg.plan_n(n)
    ws = rg.new_workspace(p, M, N, K)
    for s_ in (seed, seed + 100):
        A, B = W.random_operands(s_, M, N, K, 1, 1, 20, 20)
        C = rg.gemm(p, dev(A), dev(B), workspace=ws)
        torch.cuda.synchronize()
        assert np.array_equal(C.cpu().numpy(), oracle_c(A, B, p.out_limbs_min))


def test_persistent_rounds():
    """Two whole rounds of 256 x 256 tiles per compute unit, then K parts of
    the remaining tiles: each workgroup walks its list of tiles with the
    operand ring running on from one tile into the next."""
    M, N, K = 1024, 1024, 1024
    p = rg.plan(K, 113, 113)
    tiles = p.n_primes * (M // 256) * (N // 256)
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    print(f"persistent: M={M} N={N} K={K} n={p.n_primes} tiles={tiles} cus={cus}", flush=True)
    assert tiles > 2 * cus or cus > 256
    A, B = W.random_operands(37, M, N, K, 2, 2, 113, 113)
    p, ws, C = run_gemm(A, B, 113, 113)
    assert rg.status(ws) == 0
    assert np.array_equal(C, oracle_c(A, B, p.out_limbs_min))


def test_persistent_uneven_rounds_all_primes():
    """54 primes (q = 2 among them) on large tiles, with a last round that
    only some workgroups run: the per-prime products against the oracle's
    stage definition for q = 2 and a spread of other primes."""
    M, N, K = 768, 768, 256
    rng = np.random.default_rng(71)
    p = rg.plan_n(54)
    ps = list(p.primes)
    print(f"persistent batched: M={M} N={N} K={K} tiles={54 * 9}", flush=True)
    A_res = W.balanced_residue_planes(rng, ps, M, K)
    r = rng.integers(-(1 << 34), 1 << 34, size=(K, N), endpoint=True)
    ws = rg.new_workspace(p, M, N, K, True, "cuda")
    B = dev(r[..., None])
    rg.split(p, None, B, ws, M=M)
    rg.residue_products(p, M, N, K, ws, A_res=dev(A_res))
    torch.cuda.synchronize()
    Yp = rg.workspace_planes(p, ws, M, N, K, batched=True)["Y"].cpu().numpy()
    for j in (0, 1, 17, 30, 52, 53):
        q = ps[j]
        refB = O.residue_planes(r.T, [q])[0]
        assert np.array_equal(Yp[j, :M, :N], O.residue_product(A_res[j], refB.T, q)), f"prime {q}"


def test_output_limbs_sign_extension():
    A, B = W.random_operands(21, 40, 30, 50, 1, 1, 30, 30)
    p, ws, C = run_gemm(A, B, 30, 30, out_limbs=5)
    ref = oracle_c(A, B, 5)
    assert np.array_equal(C, ref)


def test_output_only_8_byte_aligned():
    """An output that starts 8 bytes into its allocation (even limb count):
    the reconstruction falls back from 16-byte to 8-byte limb stores."""
    A, B = W.random_operands(23, 70, 45, 60, 2, 2, 90, 90)
    p = rg.plan(60, 90, 90)
    lc = 4
    assert p.out_limbs_min <= lc
    buf = torch.full((70 * 45 * lc + 1,), 5, dtype=torch.int64, device="cuda")
    out = buf[1:].view(70, 45, lc)
    assert out.data_ptr() % 16 == 8
    rg.gemm(p, dev(A), dev(B), out_limbs=lc, out=out)
    torch.cuda.synchronize()
    assert int(buf[0]) == 5
    assert np.array_equal(out.cpu().numpy(), oracle_c(A, B, lc))


def test_k_zero_and_empty():
    p = rg.plan(0, 10, 10)
    A = torch.zeros((5, 0, 1), dtype=torch.int64, device="cuda")
    B = torch.zeros((0, 7, 1), dtype=torch.int64, device="cuda")
    C = torch.full((5, 7, 1), 123, dtype=torch.int64, device="cuda")
    rg.gemm(p, A, B, out=C, workspace=torch.empty(1, dtype=torch.uint8, device="cuda"))
    torch.cuda.synchronize()
    assert not C.any()
    A = torch.zeros((0, 4, 1), dtype=torch.int64, device="cuda")
    B = torch.zeros((4, 3, 1), dtype=torch.int64, device="cuda")
    C = rg.gemm(rg.plan(4, 3, 3), A, B)
    assert C.shape == (0, 3, 1)


def test_extreme_operands_tight_bound():
    # every entry at -2^a and -2^b: C = K * 2^(a+b) = the bound itself
    for (K, a, b, la, lb) in [(64, 20, 20, 1, 1), (4096, 100, 100, 2, 2), (300, 62, 62, 1, 1),
                              (1000, 200, 120, 4, 2)]:
        M, N = 3, 5
        Av = np.full((M, K), -(2 ** a), dtype=object)
        Bv = np.full((K, N), -(2 ** b), dtype=object)
        Av[1, :] = 2 ** a
        Bv[:, 2] = 2 ** b
        A, B = O.encode_array(Av, la), O.encode_array(Bv, lb)
        p, ws, C = run_gemm(A, B, a, b)
        got = O.decode_array(C)
        assert np.array_equal(got, Av.dot(Bv))
        assert got[0, 0] == K * 2 ** (a + b)
        assert rg.status(ws) == 0


def test_int32_accumulator_edge():
    # K = 2^17 with every residue mod 251 equal to +125: the int32 sum reaches
    # 2^17 * 125^2 = 2.048e9, the largest the accumulator must hold.
    K = 2 ** 17
    A = np.full((2, K, 1), 125, dtype=np.int64)
    B = np.full((K, 3, 1), 125, dtype=np.int64)
    B[:, 1, 0] = -125
    A[1, ::2, 0] = 376          # 376 = 125 mod 251, other primes differ
    p, ws, C = run_gemm(A, B, 9, 7)
    Av, Bv = O.decode_array(A), O.decode_array(B)
    assert np.array_equal(O.decode_array(C), Av.dot(Bv))


def test_status_flags_out_of_bound():
    A, B = W.random_operands(31, 20, 20, 40, 1, 1, 20, 20)
    p = rg.plan(40, 20, 20)
    A2 = A.copy()
    A2[3, 7, 0] = 2 ** 20 + 1          # exceeds |a| <= 2^20
    ws = rg.new_workspace(p, 20, 20, 40)
    rg.gemm(p, dev(A2), dev(B), workspace=ws)
    assert rg.status(ws) == rg.FLAG_A_RANGE
    B2 = B.copy()
    B2[0, 0, 0] = -(2 ** 20) - 1
    rg.gemm(p, dev(A), dev(B2), workspace=ws)
    assert rg.status(ws) == rg.FLAG_B_RANGE
    A3 = A.copy()
    A3[0, 0, 0] = 2 ** 20               # exactly at the bound: allowed
    A3[0, 1, 0] = -(2 ** 20)
    rg.gemm(p, dev(A3), dev(B), workspace=ws)
    assert rg.status(ws) == 0


def test_deterministic_bytes():
    A, B = W.random_operands(41, 300, 300, 300, 2, 2, 100, 100)
    p = rg.plan(300, 100, 100)
    ws = rg.new_workspace(p, 300, 300, 300)
    Ad, Bd = dev(A), dev(B)
    C1 = rg.gemm(p, Ad, Bd, workspace=ws).clone()
    C2 = rg.gemm(p, Ad, Bd, workspace=ws)
    torch.cuda.synchronize()
    assert torch.equal(C1, C2)


# ---------------------------------------------------------------------------
# batched residue (lift step)
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("M,N,K,n,seed", [(128, 16, 256, 54, 51), (100, 7, 70, 54, 52),
                                          (256, 40, 192, 20, 53), (64, 1, 64, 1, 54)])
def test_batched_residue_small(M, N, K, n, seed):
    print(f"batched M={M} N={N} K={K} n={n}", flush=True)
    rng = np.random.default_rng(seed)
    p = rg.plan_n(n)
    A_res = W.balanced_residue_planes(rng, p.primes, M, K)
    r = rng.integers(-(1 << 34), 1 << 34, size=(K, N), endpoint=True)
    ws0 = rg.new_workspace(p, M, N, K, True)
    X = rg.gemm_batched_residue(p, dev(A_res), dev(r[..., None]), workspace=ws0).cpu().numpy()
    ref = O.residue_gemm_via_crt(A_res, r, list(p.primes))
    assert np.array_equal(O.decode_array(X), ref)
    assert rg.status(ws0) == 0          # a readable status header: no bound on r, no flags


def _planted(n, values, prime_powers=False):
    """Batched call with K = 1 and B = 1: entry m of the output is the CRT
    value of the residues planted in A_res[:, m, 0], i.e. values[m]."""
    p = rg.plan_n(n, prime_powers=prime_powers)
    ps = list(p.primes)
    M = len(values)
    A_res = np.zeros((n, M, 1), dtype=np.int8)
    for j, q in enumerate(ps):
        for m, X in enumerate(values):
            A_res[j, m, 0] = (O.balanced(X, q) + 128) % 256 - 128   # as an int8 byte (128 -> -128 mod 256)
    B = np.ones((1, 1, 1), dtype=np.int64)
    return p, ps, dev(A_res), dev(B)


def _boundary_values(ps, rng, count=40):
    P = O.prod(ps)
    lo = -(P // 2) + (1 if P % 2 == 0 else 0)      # the smallest value of (-P/2, P/2]
    hi = P // 2
    vals = [0, 1, -1, hi, lo, hi - 1, lo + 1, hi - 2, lo + 2, P // 3, -(P // 3), P // 4, -(P // 4)]
    assert all(2 * v <= P and 2 * v > -P for v in vals)
    for _ in range(count):
        d = int(rng.integers(0, min(1 << 20, (P - 1) // 2)))
        vals += [hi - d, lo + d]
        x = int.from_bytes(rng.bytes(48), "little") % P - P // 2
        vals.append(x if 2 * x > -P else x + P)
    assert all(2 * v <= P and 2 * v > -P for v in vals)
    return vals


@pytest.mark.parametrize("n", [1, 2, 6, 16, 29, 30, 31, 32, 33, 47, 53, 54])
def test_reconstruct_planted_values(n):
    """Both reconstructions return the planted value, including both ends of
    (-P/2, P/2] and values next to them, for prime counts around the CRT
    kernel's one/two K-step and N-block sizes (odd and even P)."""
    rng = np.random.default_rng(1000 + n)
    ps = rg.plan_n(n).primes
    vals = _boundary_values(list(ps), rng)
    print(f"planted n={n} entries={len(vals)}", flush=True)
    p, ps, A_res, B = _planted(n, vals)
    M = len(vals)
    for method in ("crt", "garner"):
        ws = rg.new_workspace(p, M, 1, 1, True, B.device)
        rg.split(p, None, B, ws, M=M)
        rg.residue_products(p, M, 1, 1, ws, A_res=A_res)
        out = torch.full((M, 1, p.out_limbs_min + 1), 7, dtype=torch.int64, device=B.device)
        rg.reconstruct(p, M, 1, 1, ws, out, batched=True, method=method)
        got = O.decode_array(out.cpu().numpy())[:, 0]
        assert [int(v) for v in got] == vals, method


@pytest.mark.parametrize("n", [1, 2, 17, 31, 32, 33, 53, 54])
def test_reconstruct_planted_values_prime_powers(n):
    """The same with the prime-power moduli (256 first; P even): both ends
    of (-P/2, P/2] through the CRT kernel and Garner."""
    rng = np.random.default_rng(2000 + n)
    ps = rg.plan_n(n, prime_powers=True).primes
    vals = _boundary_values(list(ps), rng)
    print(f"planted prime powers n={n} entries={len(vals)}", flush=True)
    p, ps, A_res, B = _planted(n, vals, prime_powers=True)
    M = len(vals)
    for method in ("crt", "garner"):
        ws = rg.new_workspace(p, M, 1, 1, True, B.device)
        rg.split(p, None, B, ws, M=M)
        rg.residue_products(p, M, 1, 1, ws, A_res=A_res)
        out = torch.full((M, 1, p.out_limbs_min + 1), 7, dtype=torch.int64, device=B.device)
        rg.reconstruct(p, M, 1, 1, ws, out, batched=True, method=method)
        got = O.decode_array(out.cpu().numpy())[:, 0]
        assert [int(v) for v in got] == vals, method


# The quad form of the CRT kernel takes outputs of at least 1024 x 128
# entries: row groups of 128 columns (N = 1024) or flat quads (N = 1000).  It
# stages a lane's four entries in groups of G = 4 below 40 bytes per entry
# (n + 8 c_limbs) and of G = 2 from there; n + 2 > 32 slots take two K steps,
# more than 32 balanced base-256 digits of 256 P two digit blocks; c_limbs
# even stores 1 KiB runs, odd stores each limb directly.
QUAD_PLANTED = [
    # n, N, extra output limbs beyond the fewest
    (1, 1024, 0),      # G = 4, rows, direct stores
    (6, 1000, 1),      # G = 4, flat, runs
    (16, 1024, 0),     # G = 4 (32 bytes), rows, runs
    (16, 1000, 1),     # G = 2 (40 bytes), flat, direct stores
    (29, 1024, 0),     # G = 2, rows, runs
    (29, 1000, 1),     # G = 2, flat, direct stores
    (31, 1024, 1),     # two K steps
    (33, 1000, 0),     # two K steps, 32 digits (one block)
    (54, 1024, 0),     # all 54 primes (P even): two K steps, two digit blocks
    (54, 1000, 1),
]


@pytest.mark.parametrize("n,N,extra", QUAD_PLANTED)
def test_reconstruct_planted_values_quad_form(n, N, extra):
    """The planted values through the quad form: column j holds s_j times
    the planted value of its row, s_j = +1 or -1 at random (+1 throughout
    when P is even, where the negated lower end would leave (-P/2, P/2]), so
    both ends of the range and their neighbours reach every entry position of
    a lane.  Expected limbs come from the oracle's encoding of the values."""
    rng = np.random.default_rng(3000 + n)
    p = rg.plan_n(n)
    ps = list(p.primes)
    vals = _boundary_values(ps, rng)
    M = len(vals)
    assert M * N >= 1024 * 128
    signs = rng.choice([-1, 1], size=N) if O.prod(ps) % 2 else np.ones(N, dtype=np.int64)
    L = p.out_limbs_min + extra
    print(f"planted quad form n={n} M={M} N={N} limbs={L}", flush=True)
    _, _, A_res, _ = _planted(n, vals)
    B = dev(signs.astype(np.int64).reshape(1, N, 1))
    ws = rg.new_workspace(p, M, N, 1, True, B.device)
    rg.split(p, None, B, ws, M=M)
    rg.residue_products(p, M, N, 1, ws, A_res=A_res)
    out = torch.full((M, N, L), 7, dtype=torch.int64, device=B.device)
    rg.reconstruct(p, M, N, 1, ws, out, batched=True)
    got = out.cpu().numpy()
    pos = O.encode_array(np.array(vals, dtype=object), L)
    neg = O.encode_array(np.array([-v for v in vals], dtype=object), L)
    want = np.where((signs > 0)[None, :, None], pos[:, None, :], neg[:, None, :])
    assert np.array_equal(got, want)


@pytest.mark.parametrize("M,N,K,la,lb,ab,bb,seed", [(40, 33, 512, 3, 3, 170, 170, 81),
                                                    (300, 270, 200, 3, 3, 172, 168, 82),
                                                    (64, 64, 64, 2, 2, 100, 100, 83)])
def test_prime_power_products_beyond_the_primes(M, N, K, la, lb, ab, bb, seed):
    """Bounds beyond the 335-bit capacity of the primes, on the prime-power
    moduli (up to 362.8 bits): exact against the oracle, CRT and Garner."""
    print(f"prime powers M={M} N={N} K={K} bits={ab},{bb}", flush=True)
    p = rg.plan(K, ab, bb, prime_powers=True)
    assert p.primes[0] == 256 and list(p.primes) == O.moduli_set_for_bound(K, ab, bb, prime_powers=True)
    A, B = W.random_operands(seed, M, N, K, la, lb, ab, bb)
    ws = rg.new_workspace(p, M, N, K)
    C = rg.gemm(p, dev(A), dev(B), workspace=ws)
    torch.cuda.synchronize()
    ref = oracle_c(A, B, p.out_limbs_min)
    assert np.array_equal(C.cpu().numpy(), ref)
    assert rg.status(ws) == 0
    out = torch.zeros_like(C)
    rg.reconstruct(p, M, N, K, ws, out, method="garner")
    torch.cuda.synchronize()
    assert np.array_equal(out.cpu().numpy(), ref)
    planes = rg.workspace_planes(p, ws, M, N, K)
    Av, Bv = O.decode_array(A), O.decode_array(B)
    refA = O.residue_planes(Av, [256])[0]
    assert np.array_equal(planes["A"].cpu().numpy()[0, :M, :K], refA)
    refB = O.residue_planes(Bv.T, [256])[0]
    refY = O.residue_product(refA, refB.T, 256)
    assert np.array_equal(planes["Y"].cpu().numpy()[0, :M, :N], refY)


def test_prime_power_int32_edge():
    """K = 2^17 - 1 with every residue mod 256 equal to -128: the int32
    accumulator of that plane reaches 2^31 - 2^14."""
    K = 2 ** 17 - 1
    p = rg.plan_n(3, prime_powers=True)
    assert p.primes[0] == 256 and p.k_max == K
    M, N = 4, 3
    A_res = np.full((3, M, K), -128, dtype=np.int8)
    A_res[1:] = 5
    r = np.full((K, N), -128, dtype=np.int64)
    ws0 = rg.new_workspace(p, M, N, K, True)
    X = rg.gemm_batched_residue(p, dev(A_res), dev(r[..., None]), workspace=ws0).cpu().numpy()
    ref = O.residue_gemm_via_crt(A_res, r, list(p.primes))
    assert np.array_equal(O.decode_array(X), ref)
    assert rg.status(ws0) == 0          # a readable status header: no bound on r, no flags


@pytest.mark.parametrize("M,N,K,la,lb,ab,bb,seed", [SMALL[1], SMALL[3], SMALL[7],
                                                    (200, 150, 96, 3, 3, 150, 160, 71)])
def test_crt_matches_garner(M, N, K, la, lb, ab, bb, seed):
    """The two reconstructions agree bit for bit on the same Y planes."""
    print(f"crt vs garner M={M} N={N} K={K}", flush=True)
    A, B = W.random_operands(seed, M, N, K, la, lb, ab, bb)
    p, ws, C = run_gemm(A, B, ab, bb, out_limbs=8)
    out = torch.zeros((M, N, 8), dtype=torch.int64, device="cuda")
    rg.reconstruct(p, M, N, K, ws, out, method="garner")
    torch.cuda.synchronize()
    assert np.array_equal(out.cpu().numpy(), C)
    assert np.array_equal(C, oracle_c(A, B, 8))


def test_batched_residue_any_int8_and_extremes():
    rng = np.random.default_rng(61)
    p = rg.plan_n(54)
    M, N, K = 8, 8, 2 ** 17
    A_res = np.full((54, M, K), -128, dtype=np.int8)
    A_res[:, 1::2, :] = 127
    A_res[:, 5, :] = rng.integers(-128, 128, size=(54, K), dtype=np.int64).astype(np.int8)
    r = np.full((K, N), 125, dtype=np.int64)
    r[:, 3] = -(2 ** 63)
    r[:, 4] = 2 ** 63 - 1
    r[::3, 5] = rng.integers(-(2 ** 62), 2 ** 62, size=r[::3, 5].shape)
    ws0 = rg.new_workspace(p, M, N, K, True)
    X = rg.gemm_batched_residue(p, dev(A_res), dev(r[..., None]), workspace=ws0).cpu().numpy()
    ref = O.residue_gemm_via_crt(A_res, r, list(p.primes))
    assert np.array_equal(O.decode_array(X), ref)
    assert rg.status(ws0) == 0          # a readable status header: no bound on r, no flags


# The skinny right-hand side (N <= 16, one limb, K a multiple of 16 up to
# 2^16) takes the one-kernel step (products on r's bytes, residues, CRT):
# ragged rows (not a multiple of the 4-row workgroups), every column count,
# K not a multiple of the 64-wide chunks nor of the 4-chunk loop groups,
# more K chunks than workgroups and the reverse, all 54 primes or a few,
# the prime-power moduli (256 included), any int8 plane values and
# right-hand sides at the int64 ends.
SKINNY = [
    # M, N, K, n, prime_powers, seed
    (1, 1, 16, 1, False, 91),
    (100, 16, 1024, 54, False, 92),
    (300, 7, 48, 20, False, 93),
    (513, 16, 1040, 54, False, 94),
    (256, 3, 4096, 54, False, 95),
    (777, 16, 208, 54, True, 96),
    (64, 1, 4096, 6, True, 97),
    (33, 5, 4112, 20, True, 98),
    (6, 16, 12352, 54, False, 99),
]


@pytest.mark.parametrize("M,N,K,n,pp,seed", SKINNY)
def test_batched_residue_skinny_fused(M, N, K, n, pp, seed):
    print(f"skinny fused M={M} N={N} K={K} n={n} prime_powers={pp}", flush=True)
    rng = np.random.default_rng(seed)
    p = rg.plan_n(n, prime_powers=pp)
    A_res = rng.integers(-128, 128, size=(n, M, K), dtype=np.int64).astype(np.int8)
    r = rng.integers(-(1 << 62), 1 << 62, size=(K, N), dtype=np.int64)
    r[0, :] = -(2 ** 63)
    r[-1, :] = 2 ** 63 - 1
    r[1::5, :] = rng.integers(-(1 << 34), 1 << 34, size=r[1::5, :].shape, endpoint=True)
    ws0 = rg.new_workspace(p, M, N, K, True)
    X = rg.gemm_batched_residue(p, dev(A_res), dev(r[..., None]), workspace=ws0).cpu().numpy()
    ref = O.residue_gemm_via_crt(A_res, r, list(p.primes))
    assert np.array_equal(O.decode_array(X), ref)
    assert rg.status(ws0) == 0          # a readable status header: no bound on r, no flags
    # the stage calls (split, general product kernel, reconstruction) agree bit for bit
    ws = rg.new_workspace(p, M, N, K, True)
    Ad, rd = dev(A_res), dev(r[..., None])
    out = torch.empty((M, N, p.out_limbs_min), dtype=torch.int64, device="cuda")
    rg.split(p, None, rd, ws, M=M)
    rg.residue_products(p, M, N, K, ws, A_res=Ad)
    rg.reconstruct(p, M, N, K, ws, out, batched=True)
    assert np.array_equal(out.cpu().numpy(), X)


# The fused step on r of every width from 1 to 8 signed bytes, with both
# ends of the width present, and on a one-byte r with a single entry of that
# width anywhere: the byte products of r's sign-extension bytes carry the
# sign whatever the width.
@pytest.mark.parametrize("B", range(1, 9))
def test_batched_residue_skinny_byte_widths(B):
    print(f"skinny fused, r of {B} signed bytes", flush=True)
    rng = np.random.default_rng(300 + B)
    lo, hi = -(2 ** (8 * B - 1)), 2 ** (8 * B - 1) - 1
    for M, N, K, n, pp in ((130, 16, 1024, 54, False), (37, 5, 208, 20, True)):
        p = rg.plan_n(n, prime_powers=pp)
        A_res = rng.integers(-128, 128, size=(n, M, K), dtype=np.int64).astype(np.int8)
        r = rng.integers(lo, hi, size=(K, N), dtype=np.int64)
        r[0, 0], r[K - 1, N - 1] = lo, hi
        ws0 = rg.new_workspace(p, M, N, K, True)
        X = rg.gemm_batched_residue(p, dev(A_res), dev(r[..., None]), workspace=ws0).cpu().numpy()
        assert np.array_equal(O.decode_array(X), O.residue_gemm_via_crt(A_res, r, list(p.primes)))
        # one entry of this width in an otherwise one-byte r
        r1 = rng.integers(-128, 128, size=(K, N), dtype=np.int64)
        r1[rng.integers(0, K), rng.integers(0, N)] = lo if B % 2 else hi
        X1 = rg.gemm_batched_residue(p, dev(A_res), dev(r1[..., None]), workspace=ws0).cpu().numpy()
        assert np.array_equal(O.decode_array(X1), O.residue_gemm_via_crt(A_res, r1, list(p.primes)))
        assert rg.status(ws0) == 0


def test_batched_residue_skinny_int32_edge():
    """K = 2^16 with every plane entry -128 and r = -2^63 (every flipped byte
    -128): each of the nine int32 byte products reaches 2^30."""
    K = 2 ** 16
    p = rg.plan_n(54)
    M, N = 5, 3
    A_res = np.full((54, M, K), -128, dtype=np.int8)
    A_res[:, 2, :] = 127
    r = np.full((K, N), -(2 ** 63), dtype=np.int64)
    r[:, 1] = 2 ** 63 - 1
    ws0 = rg.new_workspace(p, M, N, K, True)
    X = rg.gemm_batched_residue(p, dev(A_res), dev(r[..., None]), workspace=ws0).cpu().numpy()
    ref = O.residue_gemm_via_crt(A_res, r, list(p.primes))
    assert np.array_equal(O.decode_array(X), ref)
    assert rg.status(ws0) == 0


# ---------------------------------------------------------------------------
# the five workloads at full size
# ---------------------------------------------------------------------------
FREIVALDS_P = 33554393   # the largest prime below 2^25: every product below 2^50, sums below 2^62


def mod_p_limbs(x, p=FREIVALDS_P):
    """int64 limbs [..., L] -> each value mod p (numpy int64), exactly."""
    L = x.shape[-1]
    acc = np.mod(x[..., L - 1], p)
    w = (1 << 64) % p
    for l in range(L - 2, -1, -1):
        acc = np.mod(acc * w + np.mod(x[..., l].view(np.uint64), np.uint64(p)).astype(np.int64), p)
    return acc


def freivalds_mod(Am, Bm, Cm, seed, p=FREIVALDS_P):
    """(A @ B) @ v == C @ v (mod p) for two random v; operands already reduced mod p."""
    rng = np.random.default_rng(seed)
    for _ in range(2):
        v = rng.integers(0, p, size=Cm.shape[1], dtype=np.int64)
        lhs = np.mod(Am @ np.mod(Bm @ v, p), p)
        rhs = np.mod(Cm @ v, p)
        if not np.array_equal(lhs, rhs):
            return False
    return True


def test_freivalds_helper_catches_one_wrong_entry():
    A, B = W.random_operands(5, 60, 50, 70, 2, 2, 100, 100)
    C = oracle_c(A, B, 4)
    assert freivalds_mod(mod_p_limbs(A), mod_p_limbs(B), mod_p_limbs(C), 1)
    Cv = O.decode_array(C)
    assert np.array_equal(mod_p_limbs(C), np.mod(Cv, FREIVALDS_P).astype(np.int64))
    Cv[7, 9] += 1
    assert not freivalds_mod(mod_p_limbs(A), mod_p_limbs(B), mod_p_limbs(O.encode_array(Cv, 4)), 1)


DIGESTS = json.load(open(os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden",
                                    "workload_digests.json")))


def sha256(a):
    return hashlib.sha256(np.ascontiguousarray(a).tobytes()).hexdigest()


def check_digest(name, C, inputs):
    """The output's SHA-256 equals the oracle's stored digest (inputs too)."""
    d = DIGESTS[name]
    for k, arr in inputs.items():
        assert sha256(arr) == d["inputs_sha256"][k], f"{name}: input {k} differs from the digest's"
    got = sha256(C)
    print(f"{name}: output sha256 {got} (oracle digest {d['C_sha256']})", flush=True)
    assert C.shape == (d["M"], d["N"], d["out_limbs"])
    assert got == d["C_sha256"]


def test_workload_tiny():
    wl = W.make("tiny")
    p, ws, C = run_gemm(wl.A, wl.B, wl.a_bits, wl.b_bits)
    assert p.n_primes == 6
    Av, Bv = O.decode_array(wl.A), O.decode_array(wl.B)
    ref = np.array(O.int_matmul(Av.tolist(), Bv.tolist()), dtype=object)
    assert np.array_equal(O.decode_array(C), ref)
    check_digest("tiny", C, {"A": wl.A, "B": wl.B})


def test_workload_square():
    wl = W.make("square")
    p, ws, C = run_gemm(wl.A, wl.B, wl.a_bits, wl.b_bits)
    assert p.n_primes == 10 and C.shape[-1] == 2
    ref = oracle_c(wl.A, wl.B, 2)
    assert np.array_equal(C, ref)
    check_digest("square", C, {"A": wl.A, "B": wl.B})


@pytest.mark.parametrize("name,nprimes", [("enclosure", 16), ("wide", 29)])
def test_workload_large_full(name, nprimes):
    """Every entry of the full-size product against the C oracle (OpenMP over
    rows), and the output's SHA-256 against the oracle's digest."""
    print(f"workload {name}", flush=True)
    wl = W.make(name)
    p, ws, C = run_gemm(wl.A, wl.B, wl.a_bits, wl.b_bits)
    assert p.n_primes == nprimes
    assert rg.status(ws) == 0
    check_digest(name, C, {"A": wl.A, "B": wl.B})
    ref = oracle_c(wl.A, wl.B, C.shape[-1])
    assert np.array_equal(C, ref)
    assert freivalds_mod(mod_p_limbs(wl.A), mod_p_limbs(wl.B), mod_p_limbs(C), 3)


def test_workload_dixon():
    p = rg.plan_n(54)
    wl = W.make("dixon", primes=list(p.primes))
    X = rg.gemm_batched_residue(p, dev(wl.A_res), dev(wl.B)).cpu().numpy()
    assert X.shape == (1024, 16, 6)
    ref = O.residue_gemm_via_crt(wl.A_res, wl.B[..., 0], O.primes_largest_first())
    assert np.array_equal(O.decode_array(X), ref)
    check_digest("dixon", X, {"A_res": wl.A_res, "B": wl.B})
