"""Parity of the sliced product (operands beyond the residue capacity) with the
C oracle, bit for bit (GPU only).  Operands are full-range limb arrays: every
limb uniform over 64 bits, so entries reach -2^(64 L - 1) and 2^(64 L - 1) - 1."""
import numpy as np
import pytest
import torch

import exact_integer_gemm_amd as rg
from oracle import cgemm
from oracle import oracle as O

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _setup():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    rg.load()
    cgemm.build()
    yield


def dev(x):
    return torch.from_numpy(np.ascontiguousarray(x)).cuda()


def full_range(rng, rows, cols, limbs):
    return rng.integers(0, 1 << 64, size=(rows, cols, limbs), dtype=np.uint64).view(np.int64)


@pytest.mark.parametrize("M,N,K,la,lb,seed", [
    (37, 29, 70, 4, 4, 1),        # 2 x 2 slice products, ragged
    (64, 130, 257, 3, 4, 2),      # uneven slices
    (33, 40, 96, 4, 1, 3),        # 3-limb slices of A against 1-limb B
    (20, 21, 50, 1, 6, 4),        # beyond four limbs
    (9, 11, 40, 8, 8, 5),         # 4 x 4 slice products, 17 output limbs
    (300, 260, 129, 2, 3, 6),     # several tiles per slice product
])
def test_sliced_product_exact(M, N, K, la, lb, seed):
    print(f"sliced M={M} N={N} K={K} la={la} lb={lb} seed={seed}", flush=True)
    rng = np.random.default_rng(100 + seed)
    A, B = full_range(rng, M, K, la), full_range(rng, K, N, lb)
    p = rg.sliced_plan(K, la, lb)
    C = rg.gemm_sliced(dev(A), dev(B), plan=p).cpu().numpy()
    ref = cgemm.gemm(A, B, p.out_limbs_min)
    assert np.array_equal(C, ref)


def test_sliced_extremes_at_the_k_limit():
    """K = 2^17 of (-2^255)(-2^255): C = 2^527 needs 9 limbs; and a mixed-sign column."""
    K, la = 1 << 17, 4
    A = np.zeros((2, K, la), dtype=np.int64)
    A[..., 3] = np.iinfo(np.int64).min                       # -2^255
    A[1, ::2, :] = -1                                        # -1 on every other k
    B = np.zeros((K, 2, la), dtype=np.int64)
    B[..., 3] = np.iinfo(np.int64).min
    B[:, 1, :3] = -1                                         # 2^192 - 1 - 2^255 ...
    B[:, 1, 3] = np.iinfo(np.int64).max                      # ... top limb 2^63 - 1
    C = rg.gemm_sliced(dev(A), dev(B)).cpu().numpy()
    ref = cgemm.gemm(A, B, rg.sliced_plan(K, la, la).out_limbs_min)
    assert np.array_equal(C, ref)
    assert int(O.decode_array(C[0:1, 0:1])[0, 0]) == K * (1 << 510)


def test_sliced_degenerate_sizes_and_errors():
    p = rg.sliced_plan(8, 4, 4)
    A = dev(np.ones((3, 0, 4), dtype=np.int64))
    B = dev(np.ones((0, 5, 4), dtype=np.int64))
    C = rg.gemm_sliced(A, B)                                 # K = 0: zeros
    assert C.shape == (3, 5, rg.sliced_plan(0, 4, 4).out_limbs_min) and int(C.abs().sum()) == 0
    with pytest.raises(rg.RnsError):
        rg.gemm_sliced(dev(np.ones((2, 8, 4), dtype=np.int64)), dev(np.ones((8, 2, 4), dtype=np.int64)),
                       out_limbs=p.out_limbs_min - 1)
