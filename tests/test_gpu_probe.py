"""The int8 matrix-core measurement aid (rns_probe_int8_mfma) computes the
products it claims to run.

Over a wave, the sum of every accumulator of v_mfma_i32_32x32x32_i8(X, Y) is
sum over k of (column sum of X at k) times (column sum of Y at k), where
lane l holds rows l % 32 and the 16 byte positions of half l / 32: the same
k for both operands, whatever order the instruction adds them in.  So the
wave's total over its 16 chains and all iterations (with the fragments XORed
between iterations as the kernel does) is a plain integer sum that numpy
reproduces, compared mod 2^32 (the accumulators are int32).
"""
import numpy as np
import pytest
import torch

import exact_integer_gemm_amd as rg

pytestmark = pytest.mark.gpu


def wave_totals_model(src: np.ndarray, workgroups: int, iters: int) -> np.ndarray:
    waves = workgroups * 4
    x = src.view(np.uint8).reshape(waves, 64, 8, 16)
    fa = [x[:, :, i, :].copy() for i in range(4)]
    fb = [x[:, :, 4 + i, :].copy() for i in range(4)]

    def colsum(f):   # [waves, 64, 16] bytes -> [waves, 2, 16] sums of the signed bytes over l32
        return f.view(np.int8).astype(np.int64).reshape(waves, 2, 32, 16).sum(axis=2)

    total = np.zeros(waves, dtype=np.int64)
    for _ in range(iters):
        sa, sb = [colsum(f) for f in fa], [colsum(f) for f in fb]
        for i in range(4):
            for j in range(4):
                total += (sb[j] * sa[i]).sum(axis=(1, 2))
        fa = [fa[i] ^ fb[(i + 1) & 3] for i in range(4)]
        sa = [colsum(f) for f in fa]
        for i in range(4):
            for j in range(4):
                total += (sa[j] * sb[i]).sum(axis=(1, 2))
        fb = [fb[i] ^ fa[(i + 3) & 3] for i in range(4)]
    return total % (1 << 32)


@pytest.mark.parametrize("workgroups,iters,seed", [(1, 1, 1), (3, 4, 2), (8, 7, 3)])
def test_mfma_probe_matches_model(workgroups, iters, seed):
    print(f"mfma probe workgroups={workgroups} iters={iters}", flush=True)
    rng = np.random.default_rng(seed)
    src = rng.integers(-128, 128, size=workgroups * 256 * 128, dtype=np.int64).astype(np.int8)
    out = rg.probe_int8_mfma(torch.from_numpy(src).cuda(), workgroups, iters)
    torch.cuda.synchronize()
    got = out.cpu().numpy().astype(np.int64).reshape(workgroups * 4, 64).sum(axis=1) % (1 << 32)
    assert np.array_equal(got, wave_totals_model(src, workgroups, iters))


def test_mfma_probe_zero_operands():
    src = torch.zeros(2 * 256 * 128, dtype=torch.int8, device="cuda")
    out = rg.probe_int8_mfma(src, 2, 5)
    torch.cuda.synchronize()
    assert int(out.abs().sum()) == 0
