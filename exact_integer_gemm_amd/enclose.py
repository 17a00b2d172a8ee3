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


def _plan_for(A64: torch.Tensor, B64: torch.Tensor, K: int, fmt: int) -> EnclosePlan:
    """Both operands' reductions, one host synchronisation, the plan."""
    dev = A64.device
    stats = torch.empty(8, dtype=torch.int32, device=dev)
    sws = torch.empty(FP_STATS_WS_BYTES, dtype=torch.uint8, device=dev)
    fp64_stats(A64, stats[0:4], sws)
    fp64_stats(B64, stats[4:8], sws)
    host = stats.cpu().tolist()                 # the one synchronisation
    return enclose_plan(K, host[0:4], host[4:8], fmt)


def _operands(A: torch.Tensor, B: torch.Tensor, ndim: int = 2):
    for t, name in ((A, "A"), (B, "B")):
        if not isinstance(t, torch.Tensor) or t.device.type != "cuda":
            raise ValueError(f"{name} must be a tensor on a GPU device")
        if t.dtype not in (torch.float32, torch.float64):
            raise TypeError(f"{name} must be float32 or float64, got {t.dtype}")
        if t.dim() != ndim:
            raise ValueError(f"{name} must have {ndim} dims, got shape {tuple(t.shape)}")
    if B.device != A.device:
        raise ValueError("A and B on different devices")
    fmt = 32 if (A.dtype == torch.float32 and B.dtype == torch.float32) else 64
    # binary32 -> binary64 is exact
    return A.to(torch.float64).contiguous(), B.to(torch.float64).contiguous(), fmt


def _run(fn_name: str, ep: EnclosePlan, M: int, N: int, K: int, A64, B64, lo, hi, workspace, stream) -> None:
    with torch.cuda.device(A64.device):
        rc = getattr(load(), fn_name)(ctypes.byref(ep.c), M, N, K, A64.data_ptr(), B64.data_ptr(),
                                      lo.data_ptr(), hi.data_ptr(), workspace.data_ptr(), workspace.numel(),
                                      stream)
    _check(rc, fn_name)


def _outputs(ep: EnclosePlan, shape, dev, M, N, K, workspace):
    dt = torch.float32 if ep.c.out_format == 32 else torch.float64
    lo = torch.empty(shape, dtype=dt, device=dev)
    hi = torch.empty(shape, dtype=dt, device=dev)
    need = workspace_size(ep, M, N, K)
    if workspace is None or workspace.numel() < need:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)
    return lo, hi, workspace


def mm_enclose(A: torch.Tensor, B: torch.Tensor, workspace: Optional[torch.Tensor] = None,
               return_plan: bool = False):
    """(lo, hi) with lo <= A @ B <= hi exactly (float32 pair if both operands
    are float32, else float64)."""
    A64, B64, fmt = _operands(A, B)
    M, K = A64.shape
    K2, N = B64.shape
    if K2 != K:
        raise ValueError(f"inner dimensions differ: {K} vs {K2}")
    ep = _plan_for(A64, B64, K, fmt)
    lo, hi, workspace = _outputs(ep, (M, N), A64.device, M, N, K, workspace)
    _run("rns_mm_enclose", ep, M, N, K, A64, B64, lo, hi, workspace, _stream_ptr(A64))
    return (lo, hi, ep) if return_plan else (lo, hi)


def mm_enclose_nt(A: torch.Tensor, Bt: torch.Tensor, workspace: Optional[torch.Tensor] = None):
    """(lo, hi) enclosing A @ Bt.T, Bt given as [N, K] (no transposed copy)."""
    A64, B64, fmt = _operands(A, Bt)
    M, K = A64.shape
    N, K2 = B64.shape
    if K2 != K:
        raise ValueError(f"inner dimensions differ: {K} vs {K2}")
    ep = _plan_for(A64, B64, K, fmt)
    lo, hi, workspace = _outputs(ep, (M, N), A64.device, M, N, K, workspace)
    _run("rns_mm_enclose_nt", ep, M, N, K, A64, B64, lo, hi, workspace, _stream_ptr(A64))
    return lo, hi


def bmm_enclose(A: torch.Tensor, B: torch.Tensor, workspace: Optional[torch.Tensor] = None):
    """[b, M, K] @ [b, K, N]: one plan for the whole batch (one host
    synchronisation), then one enclosure product per matrix on the stream."""
    A64, B64, fmt = _operands(A, B, 3)
    nb, M, K = A64.shape
    nb2, K2, N = B64.shape
    if nb2 != nb or K2 != K:
        raise ValueError(f"batch shapes differ: {tuple(A.shape)} and {tuple(B.shape)}")
    ep = _plan_for(A64, B64, K, fmt)
    lo, hi, workspace = _outputs(ep, (nb, M, N), A64.device, M, N, K, workspace)
    s = _stream_ptr(A64)
    for i in range(nb):
        _run("rns_mm_enclose", ep, M, N, K, A64[i], B64[i], lo[i], hi[i], workspace, s)
    return lo, hi


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


__all__ = ["EnclosePlan", "RnsError", "bmm_enclose", "digest", "enclose_plan", "fp64_stats",
           "fp64_to_limbs", "mm_enclose", "mm_enclose_nt", "round_outward", "width_ulps"]
