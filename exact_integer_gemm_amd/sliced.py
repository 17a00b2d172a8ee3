"""Exact integer products beyond the residue capacity (C ABI: ``include/rns_sliced.h``).

``C = gemm_sliced(A, B)`` for int64 limb operands of up to 8 limbs each: the
operands are cut at limb boundaries into slices whose pairwise products each fit
one exact residue product, and the shifted slice products are summed in two's
complement (Ozaki Scheme II paper, §5.1 and §5.2: slices trade additional GEMMs
for range).  Every step runs in the library's HIP kernels.
"""
from __future__ import annotations

import ctypes
from dataclasses import dataclass
from typing import Optional

import torch

from . import Plan, _check, _need, _SlicedPlan, _stream_ptr, load


@dataclass(frozen=True)
class SlicedPlan:
    """A slice plan (a copy of the C ``rns_sliced_plan_t``)."""
    slice: Plan
    a_limbs: int
    b_limbs: int
    sa: int
    sb: int
    na: int
    nb: int
    part_limbs: int
    out_limbs_min: int
    _c: _SlicedPlan

    @property
    def products(self) -> int:
        return self.na * self.nb


def sliced_plan(K: int, a_limbs: int, b_limbs: int) -> SlicedPlan:
    c = _SlicedPlan()
    _check(load().rns_sliced_plan(K, a_limbs, b_limbs, ctypes.byref(c)), "rns_sliced_plan")
    return SlicedPlan(Plan._from_c(c.slice), c.a_limbs, c.b_limbs, c.sa, c.sb, c.na, c.nb, c.part_limbs,
                      c.out_limbs_min, c)


def workspace_size(p: SlicedPlan, M: int, N: int, K: int) -> int:
    out = ctypes.c_size_t()
    _check(load().rns_sliced_workspace_size(ctypes.byref(p._c), M, N, K, ctypes.byref(out)),
           "rns_sliced_workspace_size")
    return out.value


def gemm_sliced(A: torch.Tensor, B: torch.Tensor, out_limbs: Optional[int] = None,
                plan: Optional[SlicedPlan] = None, workspace: Optional[torch.Tensor] = None,
                out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """C = A @ B exactly.  A int64 [M,K,la], B int64 [K,N,lb] (la, lb <= 8) -> int64 [M,N,out_limbs]."""
    _need(A, torch.int64, 3, "A")
    _need(B, torch.int64, 3, "B")
    M, K, la = A.shape
    K2, N, lb = B.shape
    if K2 != K:
        raise ValueError(f"inner dimensions differ: {K} vs {K2}")
    if B.device != A.device:
        raise ValueError("A and B on different devices")
    p = sliced_plan(K, la, lb) if plan is None else plan
    if (p.a_limbs, p.b_limbs) != (la, lb):
        raise ValueError("the plan was made for other operand limbs")
    lc = p.out_limbs_min if out_limbs is None else out_limbs
    if out is None:
        out = torch.empty((M, N, lc), dtype=torch.int64, device=A.device)
    _need(out, torch.int64, 3, "out")
    if tuple(out.shape) != (M, N, lc):
        raise ValueError("out has the wrong shape")
    if workspace is None:
        workspace = torch.empty(max(workspace_size(p, M, N, K), 1), dtype=torch.uint8, device=A.device)
    with torch.cuda.device(A.device):
        rc = load().rns_gemm_sliced(ctypes.byref(p._c), M, N, K, A.data_ptr(), B.data_ptr(), out.data_ptr(), lc,
                                    workspace.data_ptr(), workspace.numel(), _stream_ptr(A))
    _check(rc, "rns_gemm_sliced")
    return out
