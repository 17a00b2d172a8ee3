"""Enclosure of a floating-point matrix product (C ABI: ``include/rns_enclose.h``).

``lo, hi = mm_enclose(A, B)`` gives IEEE matrices with lo <= A @ B <= hi
entrywise, A @ B taken in exact real arithmetic: each operand is scaled by a
power of two into integer limbs, the integer product is exact (residues,
one INT8 product per prime, one reconstruction), and the exact result is
rounded outward once (enclosure-gemm, "Method").  Argument marshalling only:
the planning reductions, the scaling, the product and the rounding run in the
library's HIP kernels.  Planning needs the operands' exponent statistics on
the host: one synchronisation per call.
"""
from __future__ import annotations

import ctypes
import hashlib
from dataclasses import dataclass
from typing import Optional, Tuple

import torch

from . import (RnsError, _EnclosePlan, _FpStats, _check, _stream_ptr, load)

FP_STATS_WS_BYTES = 16384


@dataclass(frozen=True)
class EnclosePlan:
    """A copy of the C ``rns_enclose_plan_t``."""
    c: _EnclosePlan

    @property
    def fa(self) -> int:
        return self.c.fa

    @property
    def fb(self) -> int:
        return self.c.fb

    @property
    def q(self) -> int:
        return self.c.q

    @property
    def n_primes(self) -> int:
        return self.c.plan.n_primes

    @property
    def limbs(self) -> Tuple[int, int, int]:
        return self.c.a_limbs, self.c.b_limbs, self.c.c_limbs

    @property
    def zero(self) -> bool:
        return bool(self.c.zero)


def _need_float(t: torch.Tensor, name: str) -> None:
    if not isinstance(t, torch.Tensor) or t.device.type != "cuda":
        raise ValueError(f"{name} must be a tensor on a GPU device")
    if t.dtype not in (torch.float32, torch.float64):
        raise TypeError(f"{name} must be float32 or float64, got {t.dtype}")
    if t.dim() != 2:
        raise ValueError(f"{name} must be a matrix, got shape {tuple(t.shape)}")


def fp64_stats(X: torch.Tensor, out: Optional[torch.Tensor] = None,
               workspace: Optional[torch.Tensor] = None) -> torch.Tensor:
    """int32 [4] on the device: max leading-bit exponent, min lowest-set-bit
    exponent, any nonzero, any non-finite (asynchronous)."""
    if X.dtype != torch.float64 or not X.is_contiguous():
        raise ValueError("X must be contiguous float64")
    if out is None:
        out = torch.empty(4, dtype=torch.int32, device=X.device)
    if workspace is None:
        workspace = torch.empty(FP_STATS_WS_BYTES, dtype=torch.uint8, device=X.device)
    with torch.cuda.device(X.device):
        rc = load().rns_fp64_stats(X.data_ptr(), X.numel(), out.data_ptr(), workspace.data_ptr(),
                                   workspace.numel(), _stream_ptr(X))
    _check(rc, "rns_fp64_stats")
    return out


def _stats_c(v) -> _FpStats:
    s = _FpStats()
    s.max_msb, s.min_lsb, s.nonzero, s.nonfinite = (int(x) for x in v)
    return s


def enclose_plan(K: int, stats_a, stats_b, out_format: int = 64) -> EnclosePlan:
    """Plan from host copies of the two operands' stats (4 ints each)."""
    c = _EnclosePlan()
    a, b = _stats_c(stats_a), _stats_c(stats_b)
    _check(load().rns_enclose_plan(K, ctypes.byref(a), ctypes.byref(b), out_format, ctypes.byref(c)),
           "rns_enclose_plan")
    return EnclosePlan(c)


def workspace_size(ep: EnclosePlan, M: int, N: int, K: int) -> int:
    out = ctypes.c_size_t()
    _check(load().rns_enclose_workspace_size(ctypes.byref(ep.c), M, N, K, ctypes.byref(out)),
           "rns_enclose_workspace_size")
    return out.value


def mm_enclose(A: torch.Tensor, B: torch.Tensor, workspace: Optional[torch.Tensor] = None,
               return_plan: bool = False):
    """(lo, hi) with lo <= A @ B <= hi exactly (float32 pair if both operands
    are float32, else float64)."""
    _need_float(A, "A")
    _need_float(B, "B")
    M, K = A.shape
    K2, N = B.shape
    if K2 != K:
        raise ValueError(f"inner dimensions differ: {K} vs {K2}")
    if B.device != A.device:
        raise ValueError("A and B on different devices")
    fmt = 32 if (A.dtype == torch.float32 and B.dtype == torch.float32) else 64
    A64 = A.to(torch.float64).contiguous()      # binary32 -> binary64 is exact
    B64 = B.to(torch.float64).contiguous()
    dev = A.device
    stats = torch.empty(8, dtype=torch.int32, device=dev)
    sws = torch.empty(FP_STATS_WS_BYTES, dtype=torch.uint8, device=dev)
    fp64_stats(A64, stats[0:4], sws)
    fp64_stats(B64, stats[4:8], sws)
    host = stats.cpu().tolist()                 # the one synchronisation
    ep = enclose_plan(K, host[0:4], host[4:8], fmt)
    dt = torch.float32 if fmt == 32 else torch.float64
    lo = torch.empty((M, N), dtype=dt, device=dev)
    hi = torch.empty((M, N), dtype=dt, device=dev)
    need = workspace_size(ep, M, N, K)
    if workspace is None or workspace.numel() < need:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)
    with torch.cuda.device(dev):
        rc = load().rns_mm_enclose(ctypes.byref(ep.c), M, N, K, A64.data_ptr(), B64.data_ptr(),
                                   lo.data_ptr(), hi.data_ptr(), workspace.data_ptr(), workspace.numel(),
                                   _stream_ptr(A))
    _check(rc, "rns_mm_enclose")
    return (lo, hi, ep) if return_plan else (lo, hi)


def fp64_to_limbs(X: torch.Tensor, F: int, limbs: int) -> torch.Tensor:
    """floor(X * 2^F) as int64 limbs [..., limbs] (the library's scaling kernel)."""
    if X.dtype != torch.float64 or not X.is_contiguous() or X.device.type != "cuda":
        raise ValueError("X must be contiguous float64 on a GPU")
    out = torch.empty(tuple(X.shape) + (limbs,), dtype=torch.int64, device=X.device)
    with torch.cuda.device(X.device):
        rc = load().rns_fp64_to_limbs(X.data_ptr(), X.numel(), F, limbs, out.data_ptr(), _stream_ptr(X))
    _check(rc, "rns_fp64_to_limbs")
    return out


def round_outward(S: torch.Tensor, q: int, out_format: int = 64) -> Tuple[torch.Tensor, torch.Tensor]:
    """(lo, hi) of S * 2^-q for int64 limbs S [..., L] (the library's rounding kernel)."""
    if S.dtype != torch.int64 or not S.is_contiguous() or S.device.type != "cuda" or S.dim() < 1:
        raise ValueError("S must be contiguous int64 limbs on a GPU")
    dt = torch.float32 if out_format == 32 else torch.float64
    shape = tuple(S.shape[:-1])
    lo = torch.empty(shape, dtype=dt, device=S.device)
    hi = torch.empty(shape, dtype=dt, device=S.device)
    count = lo.numel()
    with torch.cuda.device(S.device):
        rc = load().rns_round_outward(S.data_ptr(), count, S.shape[-1], q, out_format, lo.data_ptr(),
                                      hi.data_ptr(), _stream_ptr(S))
    _check(rc, "rns_round_outward")
    return lo, hi


def _order_key(x: torch.Tensor) -> torch.Tensor:
    """Integers in the order of the IEEE values (adjacent values differ by 1)."""
    if x.dtype == torch.float64:
        b = x.contiguous().view(torch.int64)
        mag = b & 0x7FFFFFFFFFFFFFFF
    else:
        b = x.contiguous().view(torch.int32).to(torch.int64)
        mag = b & 0x7FFFFFFF
    return torch.where(b < 0, -mag, mag)


def width_ulps(lo: torch.Tensor, hi: torch.Tensor) -> torch.Tensor:
    """Representable steps from lo to hi (0: lo == hi)."""
    return _order_key(hi) - _order_key(lo)


def digest(lo: torch.Tensor, hi: torch.Tensor) -> str:
    """SHA-256 over the raw bits of lo then hi."""
    h = hashlib.sha256()
    for t in (lo, hi):
        h.update(t.detach().contiguous().cpu().numpy().tobytes())
    return h.hexdigest()


__all__ = ["EnclosePlan", "RnsError", "digest", "enclose_plan", "fp64_stats", "fp64_to_limbs",
           "mm_enclose", "round_outward", "width_ulps"]
