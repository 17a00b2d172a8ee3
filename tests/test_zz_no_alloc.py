"""rns_gemm_noalloc (the product with the library's fixed device scratch array
as its workspace) against rns_gemm with a caller workspace, bit for bit.

Two calls in a row, the second on a smaller input, so that the second runs on
whatever the first left in the shared array; both also against the C oracle.
"""
import ctypes

import numpy as np
import pytest
import torch

import exact_integer_gemm_amd as rg
import workloads as W
from oracle import cgemm

pytestmark = pytest.mark.gpu


def _run_both(seed, M, N, K, la, lb, ab, bb):
    print(f"noalloc case M={M} N={N} K={K} la={la} lb={lb} seed={seed}", flush=True)
    A, B = W.random_operands(seed, M, N, K, la, lb, ab, bb)
    p = rg.plan(K, ab, bb)
    Ad, Bd = torch.from_numpy(A).cuda(), torch.from_numpy(B).cuda()
    ref = rg.gemm(p, Ad, Bd)                     # rns_gemm with a workspace of its own
    out = torch.full((M, N, p.out_limbs_min), 0x5a5a5a5a5a5a5a5a, dtype=torch.int64, device="cuda")
    rg.gemm_noalloc(p, Ad, Bd, out)              # rns_gemm_noalloc
    torch.cuda.synchronize()
    got = out.cpu().numpy()
    assert np.array_equal(got, ref.cpu().numpy())
    assert np.array_equal(got, cgemm.gemm(A, B, p.out_limbs_min))


def test_noalloc_matches_gemm_twice_second_smaller():
    assert torch.cuda.is_available()
    rg.load()
    # first: 256 x 256 tiles (operand planes, product planes and split-tile
    # residues in the array); second: smaller, small tiles, over the leftovers
    _run_both(81, 768, 768, 320, 2, 2, 100, 100)
    _run_both(82, 70, 50, 130, 1, 2, 60, 90)


def test_noalloc_rejects_beyond_scratch():
    lib = rg.load()
    p = rg.plan(4096, 100, 100)
    c = p._c()
    size = ctypes.c_size_t()
    assert lib.rns_workspace_size(ctypes.byref(c), 2048, 2048, 4096, 0, ctypes.byref(size)) == 0
    assert size.value > (64 << 20)
    rc = lib.rns_gemm_noalloc(ctypes.byref(c), 2048, 2048, 4096, None, 2, None, 2, None, 4, None)
    assert rc == -10 and "scratch" in rg.error_string(rc)
