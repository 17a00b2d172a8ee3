"""Exact integer matrix product computed in residues, on gfx950.

A thin Python binding over ``librns_gemm.so`` (C ABI: ``include/rns_gemm.h``).
The binding only marshals arguments: every step of the product (residue split,
prime-batched INT8 MFMA products with the mod-q epilogue, and the
reconstruction: the centered CRT by rounded quotient of Ozaki Scheme II
§3.5.2 by default, balanced Garner as ``method="garner"``) runs in the
library's HIP kernels.  PyTorch provides device memory and the current stream.

    import exact_integer_gemm_amd as rg
    plan = rg.plan(K, a_bits, b_bits)          # primes for |A|<=2^a, |B|<=2^b
    C = rg.gemm(plan, A, B)                    # A int64 [M,K,la], B int64 [K,N,lb] on cuda
    plan54 = rg.plan_n(54)
    X = rg.gemm_batched_residue(plan54, A_res, r)   # A_res int8 [54,M,K]

The library must be built (``python -m exact_integer_gemm_amd._build``); there
is no fallback path: loading fails loudly when it is missing.
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass
from typing import List, Optional

# torch first: its HIP runtime (soname libamdhip64.so.7) must be the one the
# library binds to, so that both share device memory and streams.
import torch

from . import _build

RNS_MAX_PRIMES = 54
RNS_K_MAX = 1 << 17
RNS_MAX_IN_LIMBS = 4
RNS_MAX_OUT_LIMBS = 8
FLAG_A_RANGE = 1
FLAG_B_RANGE = 2

ERRORS = {0: "RNS_OK", -1: "RNS_E_ARG", -2: "RNS_E_K", -3: "RNS_E_CAPACITY",
          -4: "RNS_E_OUT_LIMBS", -5: "RNS_E_WORKSPACE", -6: "RNS_E_HIP", -7: "RNS_E_NONFINITE",
          -8: "RNS_E_RECONSTRUCT", -9: "RNS_E_HOSTLIB"}


class RnsError(RuntimeError):
    def __init__(self, code: int, what: str):
        self.code = code
        super().__init__(f"{what}: {ERRORS.get(code, code)} ({error_string(code)})")


class _Plan(ctypes.Structure):
    _fields_ = [("n_primes", ctypes.c_int32), ("out_limbs_min", ctypes.c_int32),
                ("a_bits", ctypes.c_int32), ("b_bits", ctypes.c_int32),
                ("k_max", ctypes.c_int64), ("log2_P", ctypes.c_double),
                ("primes", ctypes.c_int32 * RNS_MAX_PRIMES)]


class _SlicedPlan(ctypes.Structure):
    _fields_ = [("slice", _Plan), ("a_limbs", ctypes.c_int32), ("b_limbs", ctypes.c_int32),
                ("sa", ctypes.c_int32), ("sb", ctypes.c_int32), ("na", ctypes.c_int32), ("nb", ctypes.c_int32),
                ("part_limbs", ctypes.c_int32), ("out_limbs_min", ctypes.c_int32)]


class _Layout(ctypes.Structure):
    _fields_ = [("m_pad", ctypes.c_int64), ("n_pad", ctypes.c_int64), ("k_pad", ctypes.c_int64),
                ("k_block", ctypes.c_int64), ("y_pitch", ctypes.c_int64),
                ("a_off", ctypes.c_int64), ("b_off", ctypes.c_int64), ("y_off", ctypes.c_int64),
                ("status_off", ctypes.c_int64), ("total_bytes", ctypes.c_int64),
                ("tile_config", ctypes.c_int32), ("a_plane", ctypes.c_int64), ("b_plane", ctypes.c_int64)]


class _FpStats(ctypes.Structure):
    _fields_ = [("max_msb", ctypes.c_int32), ("min_lsb", ctypes.c_int32),
                ("nonzero", ctypes.c_int32), ("nonfinite", ctypes.c_int32)]


class _EnclosePlan(ctypes.Structure):
    _fields_ = [("plan", _Plan), ("fa", ctypes.c_int32), ("fb", ctypes.c_int32),
                ("a_bits", ctypes.c_int32), ("b_bits", ctypes.c_int32),
                ("a_limbs", ctypes.c_int32), ("b_limbs", ctypes.c_int32),
                ("c_limbs", ctypes.c_int32), ("q", ctypes.c_int32),
                ("out_format", ctypes.c_int32), ("zero", ctypes.c_int32)]


_lib = None


def library_path() -> str:
    return _build.LIB


def load() -> ctypes.CDLL:
    """Load librns_gemm.so; raises if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_build.LIB):
        raise RuntimeError(f"{_build.LIB} is missing: build it with "
                           "`python -m exact_integer_gemm_amd._build`")
    lib = ctypes.CDLL(_build.LIB)
    P, I32, I64, SZ, VP = (ctypes.POINTER(_Plan), ctypes.c_int32, ctypes.c_int64,
                           ctypes.c_size_t, ctypes.c_void_p)
    sig = {
        "rns_plan": (ctypes.c_int, [I64, I32, I32, P]),
        "rns_plan_n": (ctypes.c_int, [I32, P]),
        "rns_plan_moduli": (ctypes.c_int, [I64, I32, I32, I32, P]),
        "rns_plan_n_moduli": (ctypes.c_int, [I32, I32, P]),
        "rns_workspace_size": (ctypes.c_int, [P, I64, I64, I64, I32, ctypes.POINTER(SZ)]),
        "rns_workspace_layout": (ctypes.c_int, [P, I64, I64, I64, I32, ctypes.POINTER(_Layout)]),
        "rns_gemm": (ctypes.c_int, [P, I64, I64, I64, VP, I32, VP, I32, VP, I32, VP, SZ, VP]),
        "rns_gemm_batched_residue": (ctypes.c_int, [P, I64, I64, I64, VP, VP, I32, VP, I32, VP, SZ, VP]),
        "rns_gemm_noalloc": (ctypes.c_int, [P, I64, I64, I64, VP, I32, VP, I32, VP, I32, VP]),
        "rns_split": (ctypes.c_int, [P, I64, I64, I64, VP, I32, VP, I32, VP, SZ, VP]),
        "rns_residue_products": (ctypes.c_int, [P, I64, I64, I64, VP, VP, SZ, VP]),
        "rns_reconstruct": (ctypes.c_int, [P, I64, I64, I64, I32, VP, I32, VP, SZ, VP]),
        "rns_reconstruct_garner": (ctypes.c_int, [P, I64, I64, I64, I32, VP, I32, VP, SZ, VP]),
        "rns_status": (ctypes.c_int, [VP, VP, ctypes.POINTER(ctypes.c_uint32)]),
        "rns_error_string": (ctypes.c_char_p, [ctypes.c_int]),
        "rns_probe_int8_mfma": (ctypes.c_int, [VP, SZ, I32, I32, VP, VP]),
        "rns_fp64_stats": (ctypes.c_int, [VP, I64, VP, VP, SZ, VP]),
        "rns_enclose_plan": (ctypes.c_int, [I64, ctypes.POINTER(_FpStats), ctypes.POINTER(_FpStats), I32,
                                            ctypes.POINTER(_EnclosePlan)]),
        "rns_enclose_workspace_size": (ctypes.c_int, [ctypes.POINTER(_EnclosePlan), I64, I64, I64,
                                                      ctypes.POINTER(SZ)]),
        "rns_mm_enclose": (ctypes.c_int, [ctypes.POINTER(_EnclosePlan), I64, I64, I64, VP, VP, VP, VP, VP,
                                          SZ, VP]),
        "rns_mm_enclose_nt": (ctypes.c_int, [ctypes.POINTER(_EnclosePlan), I64, I64, I64, VP, VP, VP, VP, VP,
                                             SZ, VP]),
        "rns_fp64_to_limbs": (ctypes.c_int, [VP, I64, I32, I32, VP, VP]),
        "rns_inverse_workspace_size": (ctypes.c_int, [I32, I64, ctypes.POINTER(SZ)]),
        "rns_batched_inverse": (ctypes.c_int, [ctypes.POINTER(I32), I32, I64, VP, VP, VP, SZ, VP]),
        "rns_inverse_planes": (ctypes.c_int, [ctypes.POINTER(I32), I32, I64, ctypes.POINTER(I32), I32, VP, VP,
                                              SZ, VP]),
        "rns_plan_from_moduli": (ctypes.c_int, [ctypes.POINTER(I32), I32, I64, P]),
        "rns_lift_workspace_size": (ctypes.c_int, [P, I64, I64, ctypes.POINTER(SZ)]),
        "rns_dixon_lift": (ctypes.c_int, [P, I64, I64, VP, VP, VP, I32, VP, I32, VP, SZ, VP]),
        "rns_round_outward": (ctypes.c_int, [VP, I64, I32, I32, I32, VP, VP, VP]),
        "rns_host_bigint_available": (ctypes.c_int, []),
        "rns_pow_table": (ctypes.c_int, [VP, I32, I32, I64, VP]),
        "rns_pow2_quotient": (ctypes.c_int, [I64, VP, I32, VP, I32]),
        "rns_reduce_fractions": (ctypes.c_int, [VP, I64, I32, VP, I32, VP, VP, I32]),
        "rns_padic_chunks_workspace_size": (ctypes.c_int, [I64, I32, I64, I32, I32, ctypes.POINTER(SZ)]),
        "rns_padic_chunks": (ctypes.c_int, [VP, I64, I32, VP, I64, I32, I32, I32, VP, VP, SZ, VP]),
        "rns_chunk_modmul_workspace_size": (ctypes.c_int, [I64, I64, I64, I64, I64, I64, I64, I64,
                                                           ctypes.POINTER(SZ)]),
        "rns_chunk_modmul": (ctypes.c_int, [VP, I64, I64, VP, I64, VP, I64, VP, I64, I64, I64, I64, VP, VP, SZ,
                                            VP]),
        "rns_chunk_bound": (ctypes.c_int, [VP, I64, I64, VP, I64, VP, I32, VP, VP, VP]),
        "rns_chunk_numerators": (ctypes.c_int, [VP, I64, I64, VP, I64, VP, I32, I32, VP, I32, VP, I32, VP,
                                                I32, VP, I32]),
        "rns_sliced_plan": (ctypes.c_int, [I64, I32, I32, ctypes.POINTER(_SlicedPlan)]),
        "rns_sliced_workspace_size": (ctypes.c_int, [ctypes.POINTER(_SlicedPlan), I64, I64, I64,
                                                     ctypes.POINTER(SZ)]),
        "rns_gemm_sliced": (ctypes.c_int, [ctypes.POINTER(_SlicedPlan), I64, I64, I64, VP, VP, VP, I32, VP,
                                           SZ, VP]),
        "rns_padic_numerators": (ctypes.c_int, [VP, I32, I64, I32, VP, I64, VP, I32, VP, I32, VP, I32, VP,
                                                I32, VP, I32]),
        "rns_rational_reconstruct": (ctypes.c_int, [VP, I32, VP, I32, VP, I32, VP, I32, VP, I32, VP, I32]),
    }
    for name, (res, args) in sig.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _lib = lib
    return lib


def error_string(code: int) -> str:
    return load().rns_error_string(int(code)).decode()


def _check(code: int, what: str) -> None:
    if code != 0:
        raise RnsError(code, what)


@dataclass(frozen=True)
class Plan:
    """A prime plan (a copy of the C ``rns_plan_t``)."""
    n_primes: int
    out_limbs_min: int
    a_bits: int
    b_bits: int
    k_max: int
    log2_P: float
    primes: tuple

    def _c(self) -> _Plan:
        """The plan as the C struct, built on first use and kept: every entry
        point takes it as const, and filling its 54 moduli from Python costs
        more than a kernel launch."""
        c = self.__dict__.get("_cstruct")
        if c is None:
            c = _Plan()
            c.n_primes, c.out_limbs_min = self.n_primes, self.out_limbs_min
            c.a_bits, c.b_bits, c.k_max, c.log2_P = self.a_bits, self.b_bits, self.k_max, self.log2_P
            for i in range(RNS_MAX_PRIMES):
                c.primes[i] = self.primes[i] if i < len(self.primes) else 0
            object.__setattr__(self, "_cstruct", c)
        return c

    @staticmethod
    def _from_c(c: _Plan) -> "Plan":
        return Plan(c.n_primes, c.out_limbs_min, c.a_bits, c.b_bits, c.k_max, c.log2_P,
                    tuple(int(c.primes[i]) for i in range(c.n_primes)))


MODULI_PRIMES = 0
MODULI_PRIME_POWERS = 1


def plan(K: int, a_bits: int, b_bits: int, prime_powers: bool = False) -> Plan:
    """Fewest largest-first moduli with product > 2*K*2^(a_bits+b_bits): the
    primes below 256, or with ``prime_powers`` the factors of lcm(1..256)
    (up to 362.8 bits; K <= 2^17 - 1)."""
    c = _Plan()
    kind = MODULI_PRIME_POWERS if prime_powers else MODULI_PRIMES
    _check(load().rns_plan_moduli(K, a_bits, b_bits, kind, ctypes.byref(c)), "rns_plan_moduli")
    return Plan._from_c(c)


def plan_n(n_primes: int, prime_powers: bool = False) -> Plan:
    """The n largest moduli (primes below 256, or prime powers), with no operand bound."""
    c = _Plan()
    kind = MODULI_PRIME_POWERS if prime_powers else MODULI_PRIMES
    _check(load().rns_plan_n_moduli(n_primes, kind, ctypes.byref(c)), "rns_plan_n_moduli")
    return Plan._from_c(c)


def workspace_size(p: Plan, M: int, N: int, K: int, batched: bool = False) -> int:
    c = p._c()
    out = ctypes.c_size_t()
    _check(load().rns_workspace_size(ctypes.byref(c), M, N, K, int(batched), ctypes.byref(out)),
           "rns_workspace_size")
    return out.value


def layout(p: Plan, M: int, N: int, K: int, batched: bool = False) -> dict:
    c = p._c()
    out = _Layout()
    _check(load().rns_workspace_layout(ctypes.byref(c), M, N, K, int(batched), ctypes.byref(out)),
           "rns_workspace_layout")
    return {f: getattr(out, f) for f, _ in _Layout._fields_}


def new_workspace(p: Plan, M: int, N: int, K: int, batched: bool = False,
                  device: Optional[torch.device] = None) -> torch.Tensor:
    n = workspace_size(p, M, N, K, batched)
    return torch.empty(max(n, 1), dtype=torch.uint8, device=device or "cuda")


def _stream_ptr(t: torch.Tensor) -> int:
    return torch.cuda.current_stream(t.device).cuda_stream


def _need(t: torch.Tensor, dtype, ndim: int, name: str) -> None:
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be on a GPU device")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if t.dim() != ndim:
        raise ValueError(f"{name} must have {ndim} dims, got shape {tuple(t.shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def gemm(p: Plan, A: torch.Tensor, B: torch.Tensor, out_limbs: Optional[int] = None,
         workspace: Optional[torch.Tensor] = None, out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """C = A @ B exactly.  A int64 [M,K,la], B int64 [K,N,lb] -> int64 [M,N,out_limbs]."""
    _need(A, torch.int64, 3, "A")
    _need(B, torch.int64, 3, "B")
    M, K, la = A.shape
    K2, N, lb = B.shape
    if K2 != K:
        raise ValueError(f"inner dimensions differ: {K} vs {K2}")
    if B.device != A.device:
        raise ValueError("A and B on different devices")
    lc = p.out_limbs_min if out_limbs is None else out_limbs
    if out is None:
        out = torch.empty((M, N, lc), dtype=torch.int64, device=A.device)
    _need(out, torch.int64, 3, "out")
    if tuple(out.shape) != (M, N, lc):
        raise ValueError("out has the wrong shape")
    if workspace is None:
        workspace = new_workspace(p, M, N, K, False, A.device)
    c = p._c()
    with torch.cuda.device(A.device):
        rc = load().rns_gemm(ctypes.byref(c), M, N, K, A.data_ptr(), la, B.data_ptr(), lb,
                             out.data_ptr(), lc, workspace.data_ptr(), workspace.numel(),
                             _stream_ptr(A))
    _check(rc, "rns_gemm")
    return out


def gemm_noalloc(p: Plan, A: torch.Tensor, B: torch.Tensor, out: torch.Tensor) -> torch.Tensor:
    """C = A @ B exactly, like ``gemm``, with the library's fixed device
    scratch array as the workspace (``rns_gemm_noalloc``): no device memory is
    allocated, so ``out`` must be given.  Calls on one GPU share the array."""
    _need(A, torch.int64, 3, "A")
    _need(B, torch.int64, 3, "B")
    _need(out, torch.int64, 3, "out")
    M, K, la = A.shape
    K2, N, lb = B.shape
    if K2 != K:
        raise ValueError(f"inner dimensions differ: {K} vs {K2}")
    if B.device != A.device or out.device != A.device:
        raise ValueError("A, B and out on different devices")
    if tuple(out.shape[:2]) != (M, N):
        raise ValueError("out has the wrong shape")
    c = p._c()
    with torch.cuda.device(A.device):
        rc = load().rns_gemm_noalloc(ctypes.byref(c), M, N, K, A.data_ptr(), la, B.data_ptr(), lb,
                                     out.data_ptr(), out.shape[2], _stream_ptr(A))
    _check(rc, "rns_gemm_noalloc")
    return out


def gemm_batched_residue(p: Plan, A_res: torch.Tensor, B: torch.Tensor,
                         out_limbs: Optional[int] = None, workspace: Optional[torch.Tensor] = None,
                         out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """X = A_res[j] @ B (mod q_j) for every prime j, reconstructed in (-P/2, P/2]."""
    _need(A_res, torch.int8, 3, "A_res")
    _need(B, torch.int64, 3, "B")
    n, M, K = A_res.shape
    if n != p.n_primes:
        raise ValueError(f"A_res has {n} planes, the plan has {p.n_primes} primes")
    K2, N, lb = B.shape
    if K2 != K:
        raise ValueError(f"inner dimensions differ: {K} vs {K2}")
    lc = p.out_limbs_min if out_limbs is None else out_limbs
    if out is None:
        out = torch.empty((M, N, lc), dtype=torch.int64, device=B.device)
    _need(out, torch.int64, 3, "out")
    if tuple(out.shape) != (M, N, lc):
        raise ValueError("out has the wrong shape")
    if workspace is None:
        workspace = new_workspace(p, M, N, K, True, B.device)
    c = p._c()
    with torch.cuda.device(B.device):
        rc = load().rns_gemm_batched_residue(ctypes.byref(c), M, N, K, A_res.data_ptr(),
                                             B.data_ptr(), lb, out.data_ptr(), lc,
                                             workspace.data_ptr(), workspace.numel(),
                                             _stream_ptr(B))
    _check(rc, "rns_gemm_batched_residue")
    return out


# ---- the three stages, callable one at a time (rns_gemm runs them in order) ----
def split(p: Plan, A: Optional[torch.Tensor], B: torch.Tensor, workspace: torch.Tensor,
          M: Optional[int] = None) -> None:
    """Kernel 1: residue planes of A and B into ``workspace``.

    A = None is the batched-residue variant (only B is split); then M, the
    row count of the caller's residue planes, fixes the workspace layout.
    """
    _need(B, torch.int64, 3, "B")
    K, N, lb = B.shape
    if A is not None:
        _need(A, torch.int64, 3, "A")
        M, K2, la = A.shape
        if K2 != K:
            raise ValueError("inner dimensions differ")
    else:
        if M is None:
            raise ValueError("the batched-residue split needs M")
        la = 1
    c = p._c()
    with torch.cuda.device(B.device):
        rc = load().rns_split(ctypes.byref(c), M, N, K,
                              A.data_ptr() if A is not None else None, la, B.data_ptr(), lb,
                              workspace.data_ptr(), workspace.numel(), _stream_ptr(B))
    _check(rc, "rns_split")


def residue_products(p: Plan, M: int, N: int, K: int, workspace: torch.Tensor,
                     A_res: Optional[torch.Tensor] = None) -> None:
    """Kernel 2: per-prime INT8 products mod q from the planes in ``workspace``."""
    if A_res is not None:
        _need(A_res, torch.int8, 3, "A_res")
        if tuple(A_res.shape) != (p.n_primes, M, K):
            raise ValueError("A_res must be [n_primes, M, K]")
    c = p._c()
    with torch.cuda.device(workspace.device):
        rc = load().rns_residue_products(ctypes.byref(c), M, N, K,
                                         A_res.data_ptr() if A_res is not None else None,
                                         workspace.data_ptr(), workspace.numel(),
                                         _stream_ptr(workspace))
    _check(rc, "rns_residue_products")


def reconstruct(p: Plan, M: int, N: int, K: int, workspace: torch.Tensor, out: torch.Tensor,
                batched: bool = False, method: str = "crt") -> torch.Tensor:
    """Kernel 3: ``out`` (int64 [M,N,limbs]) from the Y planes.

    method "crt": rns_reconstruct (centered CRT by rounded quotient, the sum
    over primes on the matrix cores); "garner": rns_reconstruct_garner
    (balanced Garner digits).  Both give the same exact value.
    """
    _need(out, torch.int64, 3, "out")
    if tuple(out.shape[:2]) != (M, N):
        raise ValueError("out has the wrong shape")
    if method not in ("crt", "garner"):
        raise ValueError("method must be 'crt' or 'garner'")
    name = "rns_reconstruct" if method == "crt" else "rns_reconstruct_garner"
    c = p._c()
    with torch.cuda.device(out.device):
        rc = getattr(load(), name)(ctypes.byref(c), M, N, K, int(batched), out.data_ptr(),
                                   out.shape[2], workspace.data_ptr(), workspace.numel(),
                                   _stream_ptr(out))
    _check(rc, name)
    return out


def status(workspace: torch.Tensor) -> int:
    """Synchronises the current stream; returns the RNS_FLAG_* bits of the last call."""
    flags = ctypes.c_uint32()
    with torch.cuda.device(workspace.device):
        rc = load().rns_status(workspace.data_ptr(), _stream_ptr(workspace), ctypes.byref(flags))
    _check(rc, "rns_status")
    return flags.value


def probe_int8_mfma(src: torch.Tensor, workgroups: int, iters: int) -> torch.Tensor:
    """Measurement aid (rns_probe_int8_mfma): ``workgroups`` x 4 waves run
    ``iters`` x 32 v_mfma_i32_32x32x32_i8 on operand bytes read once from
    ``src`` (int8, at least workgroups * 32 KiB, on the device), with no
    memory traffic in the loop.  Returns the int32 [workgroups * 256]
    accumulator sums (asynchronously, on the current stream)."""
    _need(src, torch.int8, 1, "src")
    out = torch.empty(workgroups * 256, dtype=torch.int32, device=src.device)
    with torch.cuda.device(src.device):
        rc = load().rns_probe_int8_mfma(src.data_ptr(), src.numel(), workgroups, iters, out.data_ptr(),
                                        _stream_ptr(src))
    _check(rc, "rns_probe_int8_mfma")
    return out


def workspace_planes(p: Plan, workspace: torch.Tensor, M: int, N: int, K: int,
                     batched: bool = False) -> dict:
    """Views of the residue planes a call left in ``workspace`` (for inspection).

    Returns int8 tensors [n, rows, cols] under keys "A" (absent when the
    batched-residue operand was used in place), "B" (copies gathered from the
    K-blocked planes) and "Y" (a strided view), plus the layout under "layout".
    """
    L = layout(p, M, N, K, batched)
    n = p.n_primes
    ws8 = workspace.view(torch.int8)
    out = {"layout": L}
    kb = L["k_block"]

    def blocked(off, rows, pitch):
        kpad = L["k_pad"]
        v = ws8.as_strided((n, kpad // kb, rows, kb), (pitch, rows * kb, kb, 1), off)
        return v.permute(0, 2, 1, 3).reshape(n, rows, kpad)

    if L["a_off"] >= 0:
        out["A"] = blocked(L["a_off"], L["m_pad"], L["a_plane"])
    out["B"] = blocked(L["b_off"], L["n_pad"], L["b_plane"])
    out["Y"] = ws8.as_strided((n, L["m_pad"], L["n_pad"]),
                              (L["m_pad"] * L["y_pitch"], L["y_pitch"], 1), L["y_off"])
    return out


from .enclose import (EnclosePlan, bmm_enclose, digest, enclose_plan, fp64_stats,  # noqa: E402
                      fp64_to_limbs, mm_enclose, mm_enclose_nt, round_outward, width_ulps)
from .exact_solve import (batched_inverse, dixon_lift, inverse_planes, plan_from_moduli,  # noqa: E402
                    solve)
from .sliced import SlicedPlan, gemm_sliced, sliced_plan  # noqa: E402
