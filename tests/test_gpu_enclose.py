"""Parity of the enclosure path (scaling, exact product, outward rounding)
with the oracle (oracle/enclose.py), bit for bit (GPU only).

Cases follow the page's correctness list (enclosure-gemm, "Correctness"):
random operands at several shapes, K from 8 to 16384, integer operands
(lo == hi == the product), catastrophic cancellation, subnormal operands,
overflow to infinity, float32, and a full-size enclosure-shaped product on
sampled entries.  Operands whose exponent spread does not fit the fixed point
are rejected rather than bracketed loosely (the loose regime is not built).
"""
import math

import numpy as np
import pytest
import torch

import exact_integer_gemm_amd as rg
from oracle import enclose as E
import workloads as W

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _setup():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    rg.load()
    yield


def dev(x):
    return torch.from_numpy(np.ascontiguousarray(x)).cuda()


def gpu_enclose(A, B):
    lo, hi = rg.mm_enclose(dev(A), dev(B))
    torch.cuda.synchronize()
    return lo.cpu().numpy(), hi.cpu().numpy()


def same_bits(x, y):
    x = np.ascontiguousarray(x)
    y = np.ascontiguousarray(y)
    assert x.dtype == y.dtype and x.shape == y.shape
    return np.array_equal(x.view(np.uint8), y.view(np.uint8))


@pytest.mark.parametrize("M,K,N,seed", [(37, 53, 29, 1), (64, 128, 33, 2), (5, 300, 7, 3), (1, 1, 1, 4)])
def test_random_normal_operands(M, K, N, seed):
    print(f"enclose random M={M} K={K} N={N}", flush=True)
    rng = np.random.default_rng(seed)
    A = rng.standard_normal((M, K))
    B = rng.standard_normal((K, N))
    lo, hi = gpu_enclose(A, B)
    rlo, rhi = E.enclose(A, B)
    assert same_bits(lo, rlo) and same_bits(hi, rhi)
    w = rg.width_ulps(torch.from_numpy(lo), torch.from_numpy(hi))
    assert int(w.min()) >= 0 and int(w.max()) <= 1


@pytest.mark.parametrize("K", [8, 64, 1000, 16384])
def test_contraction_lengths(K):
    """The bracket stays one step wide whatever K (enclosure-gemm: the width
    does not depend on the contraction length)."""
    print(f"enclose K={K}", flush=True)
    rng = np.random.default_rng(100 + K)
    A = rng.standard_normal((3, K))
    B = rng.standard_normal((K, 2))
    lo, hi = gpu_enclose(A, B)
    rlo, rhi = E.enclose(A, B)
    assert same_bits(lo, rlo) and same_bits(hi, rhi)
    assert int(rg.width_ulps(torch.from_numpy(lo), torch.from_numpy(hi)).max()) <= 1


def test_integer_operands_are_exact():
    rng = np.random.default_rng(5)
    A = rng.integers(-2 ** 20, 2 ** 20, size=(40, 70)).astype(np.float64)
    B = rng.integers(-2 ** 20, 2 ** 20, size=(70, 30)).astype(np.float64)
    lo, hi = gpu_enclose(A, B)
    ref = (A.astype(np.int64) @ B.astype(np.int64)).astype(np.float64)
    assert np.array_equal(lo, ref) and np.array_equal(hi, ref)
    assert np.array_equal(lo, (torch.from_numpy(A) @ torch.from_numpy(B)).numpy())


def test_catastrophic_cancellation():
    A = np.array([[1e16, 1.0, -1e16, 2.0 ** -60], [1.0, 1.0, 1.0, 1.0]])
    B = np.ones((4, 3))
    B[3, 1] = -1.0
    lo, hi = gpu_enclose(A, B)
    rlo, rhi = E.enclose(A, B)
    assert same_bits(lo, rlo) and same_bits(hi, rhi)
    assert lo[0, 0] == 1.0 and hi[0, 0] == math.nextafter(1.0, 2.0)


def test_subnormal_operands_and_results():
    rng = np.random.default_rng(6)
    A = rng.standard_normal((6, 10)) * 2.0 ** -1000
    A[0, 0] = math.ldexp(1.0, -1074)                  # the smallest subnormal
    A[1, :] = rng.standard_normal(10) * 2.0 ** -1060  # subnormal entries
    B = rng.standard_normal((10, 5)) * 2.0 ** 40
    B[:, 4] = rng.standard_normal(10) * 2.0 ** -40     # products far below the subnormal range
    lo, hi = gpu_enclose(A, B)
    rlo, rhi = E.enclose(A, B)
    assert same_bits(lo, rlo) and same_bits(hi, rhi)


def test_overflow_to_infinity():
    A = np.array([[2.0 ** 1000, 3 * 2.0 ** 998], [-(2.0 ** 1000), 2.0 ** 999]])
    B = np.array([[2.0 ** 30, 1.0], [2.0 ** 25, 0.5]])
    lo, hi = gpu_enclose(A, B)
    rlo, rhi = E.enclose(A, B)
    assert same_bits(lo, rlo) and same_bits(hi, rhi)
    assert hi[0, 0] == math.inf and lo[0, 0] == np.finfo(np.float64).max
    assert lo[1, 0] == -math.inf and hi[1, 0] == -np.finfo(np.float64).max
    assert math.isfinite(lo[0, 1]) and lo[0, 1] == hi[0, 1]


def test_float32_operands():
    rng = np.random.default_rng(7)
    A = rng.standard_normal((20, 45)).astype(np.float32)
    B = rng.standard_normal((45, 12)).astype(np.float32)
    B[0, 0] = np.float32(2.0 ** -140)                 # binary32 subnormal
    lo, hi = gpu_enclose(A, B)
    assert lo.dtype == np.float32
    rlo, rhi = E.enclose(A.astype(np.float64), B.astype(np.float64), "binary32")
    assert same_bits(lo, rlo) and same_bits(hi, rhi)


def test_zero_operand_and_empty_contraction():
    A = np.zeros((4, 6))
    B = np.random.default_rng(8).standard_normal((6, 3))
    lo, hi = gpu_enclose(A, B)
    assert same_bits(lo, np.zeros((4, 3))) and same_bits(hi, np.zeros((4, 3)))
    lo, hi = gpu_enclose(np.zeros((2, 0)), np.zeros((0, 5)))
    assert same_bits(lo, np.zeros((2, 5))) and same_bits(hi, np.zeros((2, 5)))


def test_wide_spread_on_prime_power_moduli():
    """Exponent spreads whose exact product needs more than the primes'
    334.9 bits run on the prime-power moduli and stay bit-exact."""
    rng = np.random.default_rng(12)
    A = rng.standard_normal((9, 64)) * 2.0 ** rng.integers(-64, 64, size=(9, 64))
    B = rng.standard_normal((64, 7)) * 2.0 ** rng.integers(-54, 54, size=(64, 7))
    lo, hi, ep = rg.mm_enclose(dev(A), dev(B), return_plan=True)
    torch.cuda.synchronize()
    assert ep.c.plan.primes[0] == 256, "this case is meant to need the prime powers"
    rlo, rhi = E.enclose(A, B)
    assert same_bits(lo.cpu().numpy(), rlo) and same_bits(hi.cpu().numpy(), rhi)


def test_nt_variant():
    """A @ Bt.T with Bt given as [N, K] (enclosure-gemm, "Usage")."""
    rng = np.random.default_rng(13)
    A = rng.standard_normal((13, 70))
    Bt = rng.standard_normal((21, 70)) * 2.0 ** 20
    lo, hi = rg.mm_enclose_nt(dev(A), dev(Bt))
    torch.cuda.synchronize()
    rlo, rhi = E.enclose(A, Bt.T.copy())
    assert same_bits(lo.cpu().numpy(), rlo) and same_bits(hi.cpu().numpy(), rhi)


def test_batched_shares_one_plan():
    """Five 20x256x12 products under one plan (enclosure-gemm, "Measured":
    the batch pays one plan and one synchronisation)."""
    rng = np.random.default_rng(14)
    A = rng.standard_normal((5, 20, 256))
    B = rng.standard_normal((5, 256, 12))
    A[3] *= 2.0 ** -30
    lo, hi = rg.bmm_enclose(dev(A), dev(B))
    torch.cuda.synchronize()
    for i in range(5):
        rlo, rhi = E.enclose(A[i], B[i])
        assert same_bits(lo[i].cpu().numpy(), rlo) and same_bits(hi[i].cpu().numpy(), rhi), i


def test_rejected_operands():
    with pytest.raises(rg.RnsError) as e:
        rg.mm_enclose(dev(np.array([[1.0, np.nan]])), dev(np.ones((2, 2))))
    assert e.value.code == -7
    wide = np.array([[2.0 ** 300, 2.0 ** -300]])   # 600 binades: beyond the fixed point
    with pytest.raises(rg.RnsError) as e:
        rg.mm_enclose(dev(wide), dev(np.ones((2, 1))))
    assert e.value.code == -3


def test_scaling_and_rounding_kernels_alone():
    """The two conversion kernels against the oracle's definitions."""
    rng = np.random.default_rng(9)
    X = rng.standard_normal(500) * 2.0 ** rng.integers(-60, 60, size=500)
    X[:3] = [0.0, -0.0, -math.ldexp(1.0, -70)]
    F = 80
    limbs = rg.fp64_to_limbs(dev(X), F, 4).cpu().numpy()
    from oracle import oracle as O
    got = O.decode_array(limbs.reshape(500, 1, 4))[:, 0]
    ref = E.scaled_integers(X, F)
    assert [int(v) for v in got] == [int(v) for v in ref]
    S = rng.integers(-2 ** 62, 2 ** 62, size=(300, 3)).astype(np.int64)
    S[:, 2] = rng.integers(-3, 3, size=300)
    S[0] = 0
    vals = O.decode_array(S.reshape(300, 1, 3))[:, 0]
    for q in (0, 77, 1200, -900):
        lo, hi = rg.round_outward(dev(S), q)
        rlo, rhi = E.enclose_from_integer(vals, q)
        assert same_bits(lo.cpu().numpy(), rlo) and same_bits(hi.cpu().numpy(), rhi), q
        lo32, hi32 = rg.round_outward(dev(S), q, 32)
        rlo32, rhi32 = E.enclose_from_integer(vals, q, "binary32")
        assert same_bits(lo32.cpu().numpy(), rlo32) and same_bits(hi32.cpu().numpy(), rhi32), q


def test_enclosure_shape_full_size():
    """A[1024,4096] @ B[4096,1024] of N(0,1) binary64 entries: the whole (lo,
    hi) against the SHA-256 of the oracle's enclosure of every entry
    (tests/golden/enclosure_digest.json, written from oracle/ only), sampled
    entries against the live oracle, and the bracket width everywhere."""
    import hashlib
    import json
    import os
    print("enclose full size 1024x4096x1024", flush=True)
    dg = json.load(open(os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden",
                                     "enclosure_digest.json")))
    A, B = W.fp64_normal_pair(dg["seed"], dg["M"], dg["K"], dg["N"])
    assert hashlib.sha256(A.tobytes()).hexdigest() == dg["inputs_sha256"]["A"]
    assert hashlib.sha256(B.tobytes()).hexdigest() == dg["inputs_sha256"]["B"]
    lo, hi, ep = rg.mm_enclose(dev(A), dev(B), return_plan=True)
    torch.cuda.synchronize()
    print(f"plan: fa={ep.fa} fb={ep.fb} primes={ep.n_primes} limbs={ep.limbs}", flush=True)
    assert (ep.fa, ep.fb) == (dg["Fa"], dg["Fb"])
    glo_all, ghi_all = lo.cpu().numpy(), hi.cpu().numpy()
    slo = hashlib.sha256(np.ascontiguousarray(glo_all).tobytes()).hexdigest()
    shi = hashlib.sha256(np.ascontiguousarray(ghi_all).tobytes()).hexdigest()
    print(f"lo sha256 {slo} (oracle {dg['lo_sha256']}); hi sha256 {shi} (oracle {dg['hi_sha256']})", flush=True)
    w = rg.width_ulps(lo, hi)
    assert int(w.min()) >= 0 and int(w.max()) <= 1
    rng = np.random.default_rng(10)
    rows = np.sort(rng.choice(1024, size=6, replace=False))
    cols = np.sort(rng.choice(1024, size=48, replace=False))
    rlo, rhi = E.enclose(A[rows], B[:, cols])
    assert same_bits(glo_all[np.ix_(rows, cols)], rlo) and same_bits(ghi_all[np.ix_(rows, cols)], rhi)
    assert slo == dg["lo_sha256"] and shi == dg["hi_sha256"]
