"""Host-side checks of the C ABI (no GPU needed).

The library must load, export every entry point ``include/*.h`` declares, share PyTorch's HIP runtime, plan exactly like the oracle, and turn
every invalid argument into its error code before anything is launched.
"""
import ctypes
import os
import re

import pytest

import exact_integer_gemm_amd as rg
from exact_integer_gemm_amd import _build
from oracle import oracle as O

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADERS = [os.path.join(ROOT, "include", h) for h in sorted(os.listdir(os.path.join(ROOT, "include")))
           if h.endswith(".h")]


@pytest.fixture(scope="module")
def lib():
    if _build.is_stale():
        _build.build()
    return rg.load()


def declared_functions():
    names = set()
    for h in HEADERS:
        text = re.sub(r"/\*.*?\*/", "", open(h).read(), flags=re.S)
        names |= set(re.findall(r"^\s*(?:int|const char \*)\s*\*?(rns_\w+)\s*\(", text, flags=re.M))
    return sorted(names)


def test_exports_every_declared_symbol(lib):
    names = declared_functions()
    assert set(names) >= {"rns_plan", "rns_plan_n", "rns_workspace_size", "rns_gemm",
                          "rns_gemm_batched_residue", "rns_status", "rns_error_string",
                          "rns_workspace_layout", "rns_fp64_stats", "rns_enclose_plan",
                          "rns_enclose_workspace_size", "rns_mm_enclose", "rns_fp64_to_limbs",
                          "rns_round_outward"}
    for n in names:
        assert hasattr(lib, n), n
    nm = os.popen(f"nm -D --defined-only {_build.LIB}").read()
    for n in names:
        assert re.search(rf"\bT {n}\b", nm), f"{n} not exported"


def test_one_hip_runtime_in_process(lib):
    import torch  # noqa: F401  (already imported by the binding)
    maps = open("/proc/self/maps").read()
    libs = {line.split()[-1] for line in maps.splitlines() if "libamdhip64" in line}
    assert len(libs) == 1, libs


def test_plan_struct_matches_header(lib):
    # rns_plan_t: 4 int32, int64, double, int32[54]
    assert ctypes.sizeof(rg._Plan) == 4 * 4 + 8 + 8 + 4 * 54
    # rns_fp_stats_t: 4 int32; rns_enclose_plan_t: rns_plan_t then 10 int32
    assert ctypes.sizeof(rg._FpStats) == 16
    assert ctypes.sizeof(rg._EnclosePlan) == ctypes.sizeof(rg._Plan) + 10 * 4


@pytest.mark.parametrize("K,a,b", [(64, 20, 20), (1024, 31, 31), (4096, 55, 55), (4096, 100, 100),
                                   (1, 0, 0), (2 ** 17, 1, 1), (3, 150, 170), (4096, 160, 160),
                                   (1000, 7, 250), (0, 5, 5)])
def test_plan_agrees_with_oracle(lib, K, a, b):
    p = rg.plan(K, a, b)
    ps = O.prime_set_for_bound(max(K, 1), a, b)
    assert list(p.primes) == ps
    assert p.n_primes == len(ps)
    assert p.out_limbs_min == O.limbs_to_hold(O.prod(ps))
    assert p.k_max == max(K, 1) and p.a_bits == a and p.b_bits == b
    assert abs(p.log2_P - sum(__import__("math").log2(q) for q in ps)) < 1e-9


def test_plan_sweep_against_oracle(lib):
    for K in (1, 7, 64, 1000, 4096, 2 ** 17):
        for s in range(0, 334, 9):
            a, b = s // 2, s - s // 2
            try:
                ps = O.prime_set_for_bound(K, a, b)
            except ValueError:
                with pytest.raises(rg.RnsError) as e:
                    rg.plan(K, a, b)
                assert e.value.code == -3
                continue
            assert list(rg.plan(K, a, b).primes) == ps


def test_plan_n(lib):
    p = rg.plan_n(54)
    assert list(p.primes) == O.primes_largest_first()
    assert p.out_limbs_min == 6 and p.k_max == 2 ** 17 and p.a_bits == -1
    assert list(rg.plan_n(10).primes) == O.primes_largest_first()[:10]
    for bad in (0, -1, 55):
        with pytest.raises(rg.RnsError) as e:
            rg.plan_n(bad)
        assert e.value.code == -1


def test_plan_errors(lib):
    with pytest.raises(rg.RnsError) as e:
        rg.plan(2 ** 17 + 1, 1, 1)
    assert e.value.code == -2
    with pytest.raises(rg.RnsError) as e:
        rg.plan(-1, 1, 1)
    assert e.value.code == -2
    with pytest.raises(rg.RnsError) as e:
        rg.plan(4096, 170, 170)
    assert e.value.code == -3
    for a, b in ((-1, 3), (3, -1), (256, 0)):
        with pytest.raises(rg.RnsError) as e:
            rg.plan(16, a, b)
        assert e.value.code == -1
    assert lib.rns_plan(16, 1, 1, None) == -1


def test_error_strings(lib):
    for code in (0, -1, -2, -3, -4, -5, -6, 99):
        s = rg.error_string(code)
        assert isinstance(s, str) and s


def test_workspace_size_and_layout(lib):
    p = rg.plan(4096, 100, 100)
    L = rg.layout(p, 2048, 2048, 4096)
    n = p.n_primes
    assert L["m_pad"] == 2048 and L["n_pad"] == 2048 and L["k_pad"] == 4096
    # operand planes K-blocked by 64; product rows at an odd multiple of 128 bytes
    assert L["k_block"] == 64
    assert L["y_pitch"] >= 2048 and L["y_pitch"] % 128 == 0 and (L["y_pitch"] // 128) % 2 == 1
    assert L["b_off"] >= L["a_off"] + n * 2048 * 4096
    assert L["y_off"] >= L["b_off"] + n * 2048 * 4096
    assert L["total_bytes"] >= L["y_off"] + n * 2048 * L["y_pitch"]
    assert rg.workspace_size(p, 2048, 2048, 4096) == L["total_bytes"]
    # ragged shapes are padded to whole tiles
    L = rg.layout(p, 65, 70, 130)
    assert L["m_pad"] >= 65 and L["n_pad"] >= 70 and L["k_pad"] >= 130 and L["k_pad"] % 64 == 0
    # batched residue: aligned A_res is used in place
    p54 = rg.plan_n(54)
    L = rg.layout(p54, 1024, 16, 1024, batched=True)
    assert L["a_off"] == -1
    L = rg.layout(p54, 1000, 16, 1000, batched=True)
    assert L["a_off"] >= 0
    with pytest.raises(rg.RnsError) as e:
        rg.workspace_size(rg.plan(64, 20, 20), 64, 64, 65)
    assert e.value.code == -2


def _call_gemm(lib, plan, M, N, K, A=1 << 20, la=1, B=1 << 21, lb=1, C=1 << 22, lc=None,
               ws=1 << 23, ws_bytes=None):
    c = plan._c()
    lc = plan.out_limbs_min if lc is None else lc
    if ws_bytes is None:
        ws_bytes = 1 << 40
    return lib.rns_gemm(ctypes.byref(c), M, N, K, A, la, B, lb, C, lc, ws, ws_bytes, None)


def test_gemm_validation_before_launch(lib):
    # None of these reaches a launch: the pointers are never dereferenced.
    p = rg.plan(64, 20, 20)
    assert _call_gemm(lib, p, 64, 64, 64, lc=0) == -4
    assert _call_gemm(lib, p, 64, 64, 64, lc=9) == -4
    assert _call_gemm(lib, p, 64, 64, 64, la=0) == -1
    assert _call_gemm(lib, p, 64, 64, 64, lb=5) == -1
    assert _call_gemm(lib, p, -1, 64, 64) == -1
    assert _call_gemm(lib, p, 64, 64, 65) == -2          # above the plan's K
    assert _call_gemm(lib, p, 64, 64, 64, A=None) == -1
    assert _call_gemm(lib, p, 64, 64, 64, ws=None) == -1
    assert _call_gemm(lib, p, 64, 64, 64, ws_bytes=100) == -5
    assert _call_gemm(lib, p, 0, 64, 64) == 0            # empty: no-op
    assert _call_gemm(lib, p, 64, 0, 64, A=None, B=None, C=None, ws=None) == 0
    bad = p._c()
    bad.n_primes = 0
    assert lib.rns_gemm(ctypes.byref(bad), 4, 4, 4, 1, 1, 1, 1, 1, 1, 1, 1 << 30, None) == -1
    bad = p._c()
    bad.primes[1] = bad.primes[0]      # repeated prime
    assert lib.rns_gemm(ctypes.byref(bad), 4, 4, 4, 1, 1, 1, 1, 1, 1, 1, 1 << 30, None) == -1
    bad = p._c()
    bad.primes[0] = 250                # not a prime
    assert lib.rns_gemm(ctypes.byref(bad), 4, 4, 4, 1, 1, 1, 1, 1, 1, 1, 1 << 30, None) == -1


def test_batched_validation_before_launch(lib):
    p = rg.plan_n(54)
    c = p._c()
    f = lib.rns_gemm_batched_residue
    assert f(ctypes.byref(c), 8, 8, 8, None, 1, 1, 1, 6, 1, 1 << 30, None) == -1
    assert f(ctypes.byref(c), 8, 8, 8, 1, 1, 1, 1, 5, 1, 1 << 30, None) == -4
    assert f(ctypes.byref(c), 8, 8, 8, 1, 1, 0, 1, 6, 1, 1 << 30, None) == -1
    assert f(ctypes.byref(c), 8, 8, 2 ** 17 + 1, 1, 1, 1, 1, 6, 1, 1 << 30, None) == -2
    assert f(ctypes.byref(c), 8, 8, 8, 1, 1, 1, 1, 6, 1, 10, None) == -5
    assert f(ctypes.byref(c), 0, 8, 8, None, None, 1, None, 6, None, 0, None) == 0


def test_status_arguments(lib):
    assert lib.rns_status(None, None, ctypes.byref(ctypes.c_uint32())) == -1
    assert lib.rns_status(1, None, None) == -1


def test_binding_rejects_bad_tensors(lib):
    import torch
    p = rg.plan(8, 4, 4)
    A = torch.zeros((2, 8, 1), dtype=torch.int64)
    with pytest.raises(ValueError):
        rg.gemm(p, A, A.clone())          # CPU tensors are refused


# ---------------------------------------------------------------------------
# enclosure planner (host logic; enclosure-gemm, "Method")
# ---------------------------------------------------------------------------
def _stats_of(X):
    """The four planner reductions of an array, from the oracle's definitions."""
    import math
    import numpy as np
    from oracle import enclose as E
    vals = [float(x) for x in np.asarray(X, dtype=np.float64).ravel()]
    nonfinite = int(any(not math.isfinite(v) for v in vals))
    nz = [v for v in vals if math.isfinite(v) and v != 0]
    if not nz:
        return (-2 ** 31, 2 ** 31 - 1, 0, nonfinite)
    msb = max(math.frexp(v)[1] - 1 for v in nz)
    lsb = min(E.lowest_set_bit_exponent(v) for v in nz)
    return (msb, lsb, 1, nonfinite)


def test_enclose_plan_scales_like_the_oracle(lib):
    import numpy as np
    from oracle import enclose as E
    rng = np.random.default_rng(11)
    A = rng.standard_normal((6, 9)) * 2.0 ** rng.integers(-20, 20, size=(6, 9))
    B = rng.standard_normal((9, 4))
    ep = rg.enclose_plan(9, _stats_of(A), _stats_of(B), 64)
    assert ep.fa == E.coarsest_lossless_scale(A) and ep.fb == E.coarsest_lossless_scale(B)
    SA = E.scaled_integers(A, ep.fa)
    SB = E.scaled_integers(B, ep.fb)
    assert max(abs(int(v)) for v in SA.ravel()) < 2 ** ep.c.a_bits
    assert max(abs(int(v)) for v in SB.ravel()) < 2 ** ep.c.b_bits
    assert ep.q == ep.fa + ep.fb and not ep.zero
    ps = O.prime_set_for_bound(9, ep.c.a_bits, ep.c.b_bits)
    assert ep.n_primes == len(ps)


def test_enclose_plan_errors_and_zero(lib):
    import numpy as np
    with pytest.raises(rg.RnsError) as e:
        rg.enclose_plan(4, _stats_of([1.0, np.inf]), _stats_of([1.0]), 64)
    assert e.value.code == -7
    with pytest.raises(rg.RnsError) as e:
        rg.enclose_plan(4, _stats_of([2.0 ** 300, 2.0 ** -300]), _stats_of([1.0]), 64)
    assert e.value.code == -3
    with pytest.raises(rg.RnsError) as e:     # each fits 4 limbs, the product does not fit P
        rg.enclose_plan(4096, _stats_of([2.0 ** 100, 2.0 ** -90]), _stats_of([2.0 ** 100, 2.0 ** -90]), 64)
    assert e.value.code == -3
    with pytest.raises(rg.RnsError) as e:
        rg.enclose_plan(2 ** 17 + 1, _stats_of([1.0]), _stats_of([1.0]), 64)
    assert e.value.code == -2
    with pytest.raises(rg.RnsError) as e:
        rg.enclose_plan(4, _stats_of([1.0]), _stats_of([1.0]), 16)
    assert e.value.code == -1
    ep = rg.enclose_plan(5, _stats_of(np.zeros(6)), _stats_of([3.0, 1e300]), 32)
    assert ep.zero and ep.c.out_format == 32


def test_workspace_size_with_empty_contraction(lib):
    """K == 0 (no split work at all) still has a workspace size."""
    for M, N in ((2, 5), (300, 300), (1, 40)):
        assert rg.workspace_size(rg.plan(0, 0, 0), M, N, 0) >= 0
        assert rg.workspace_size(rg.plan_n(54), M, N, 0, True) >= 0


@pytest.mark.parametrize("K,a,b", [(64, 20, 20), (4096, 100, 100), (4096, 170, 170), (131071, 170, 170),
                                   (3, 180, 178), (0, 5, 5)])
def test_prime_power_plan_agrees_with_oracle(lib, K, a, b):
    p = rg.plan(K, a, b, prime_powers=True)
    ms = O.moduli_set_for_bound(max(K, 1), a, b, prime_powers=True)
    assert list(p.primes) == ms
    assert p.out_limbs_min == O.limbs_to_hold(O.prod(ms))
    assert p.k_max == max(K, 1)


def test_prime_power_plan_limits(lib):
    with pytest.raises(rg.RnsError) as e:
        rg.plan(2 ** 17, 1, 1, prime_powers=True)       # 256 needs K <= 2^17 - 1
    assert e.value.code == -2
    with pytest.raises(rg.RnsError) as e:
        rg.plan(8, 181, 181, prime_powers=True)
    assert e.value.code == -3
    p = rg.plan_n(54, prime_powers=True)
    assert p.k_max == 2 ** 17 - 1 and p.out_limbs_min == 6 and abs(p.log2_P - 362.828) < 1e-3
    # a plan whose 256 claims K up to 2^17 is refused by every entry point
    bad = rg.Plan(p.n_primes, p.out_limbs_min, -1, -1, 2 ** 17, p.log2_P, p.primes)
    with pytest.raises(rg.RnsError) as e:
        rg.workspace_size(bad, 4, 4, 4)
    assert e.value.code == -1


def test_enclose_plan_falls_back_to_prime_powers(lib):
    """Spreads whose product needs more than the primes' 334.9 bits take the
    prime-power moduli (lossless up to 362.8 bits)."""
    import numpy as np
    A = np.array([2.0 ** 100, 2.0 ** -70])       # 171-bit integers
    B = np.array([2.0 ** 90, 2.0 ** -70])        # 161-bit integers
    ep = rg.enclose_plan(64, _stats_of(A), _stats_of(B), 64)
    assert ep.c.plan.primes[0] == 256
    assert ep.c.a_bits + ep.c.b_bits + 7 > 335


def test_sliced_plan_choices():
    """Slice widths, counts and output limbs of the sliced product (host only)."""
    import exact_integer_gemm_amd as rg
    p = rg.sliced_plan(4096, 4, 4)
    assert (p.sa, p.sb, p.na, p.nb) == (2, 2, 2, 2)
    # a slice product spans 2 K 2^256 < P of its primes
    assert p.slice.log2_P > 1 + 12 + 256
    assert p.out_limbs_min == 9                 # 510 + 12 bits and a sign: 9 limbs
    p = rg.sliced_plan(70, 4, 1)
    assert (p.sa, p.sb, p.na, p.nb) == (3, 1, 2, 1)
    p = rg.sliced_plan(1 << 17, 8, 8)
    assert (p.na, p.nb, p.out_limbs_min) == (4, 4, 17)
    for bad in ((-1, 4, 4), (8, 0, 4), (8, 4, 9)):
        with pytest.raises(rg.RnsError) as e:
            rg.sliced_plan(*bad)
        assert e.value.code == -1
    with pytest.raises(rg.RnsError) as e:
        rg.sliced_plan((1 << 17) + 1, 4, 4)
    assert e.value.code == -2


def test_noalloc_rejects_before_any_device_work(lib):
    """rns_gemm_noalloc validates the plan and the sizes and refuses shapes
    whose workspace exceeds its fixed array, all on the host."""
    p = rg.plan(4096, 100, 100)
    c = p._c()
    assert lib.rns_gemm_noalloc(ctypes.byref(c), 2048, 2048, 4096, None, 2, None, 2, None, 4, None) == -10
    assert lib.rns_gemm_noalloc(None, 8, 8, 8, None, 1, None, 1, None, 1, None) == -1
    assert lib.rns_gemm_noalloc(ctypes.byref(c), 8, 8, 2 ** 17 + 1, None, 1, None, 1, None, 4, None) == -2
    assert "scratch" in lib.rns_error_string(-10).decode()


def test_mfma_probe_rejects_before_any_device_work(lib):
    """The measurement aid checks its buffer and counts before it launches."""
    E_ARG = -1
    out = ctypes.c_void_p(256)
    fake = ctypes.c_void_p(4096)            # never dereferenced: every call below is rejected
    assert lib.rns_probe_int8_mfma(None, 1 << 20, 1, 1, out, None) == E_ARG
    assert lib.rns_probe_int8_mfma(fake, 1 << 20, 1, 1, None, None) == E_ARG
    assert lib.rns_probe_int8_mfma(fake, 32 * 1024 - 1, 1, 1, out, None) == E_ARG   # one workgroup needs 32 KiB
    assert lib.rns_probe_int8_mfma(fake, 1 << 20, 0, 1, out, None) == E_ARG
    assert lib.rns_probe_int8_mfma(fake, 1 << 20, 1, 0, out, None) == E_ARG
    assert lib.rns_probe_int8_mfma(ctypes.c_void_p(4100), 1 << 20, 1, 1, out, None) == E_ARG   # unaligned

