"""The parity checks of the full-size GPU tests, exercised on the CPU: a result computed the
way the kernels compute it passes, and one planted mistake (a single reduce output two bf16
ulps off, one expert's Y block taken from the wrong expert, one h row at a block edge) fails.
Rows inside a 64-row block of a large expert are sampled at random only: a fault confined to
one such row can pass the GEMM check (the reduce check reads every element of Y it sums)."""
import numpy as np
import pytest
import torch

from oracle import moe, nvfp4
from tests.gpu_util import assert_reduce_elementwise, bf16_ulp, check_every_expert


def _reduce_like_the_kernel(y, s2r, w):
    """float32 multiply-add in ascending j, one rounding to bf16 at the end."""
    T, k = w.shape
    acc = np.zeros((T, y.shape[1]), np.float32)
    for j in range(k):
        acc = (acc + w[:, j:j + 1] * y[s2r[np.arange(T) * k + j]]).astype(np.float32)
    return torch.from_numpy(acc).to(torch.bfloat16).float().numpy()


def test_reduce_check_accepts_float32_sum_and_catches_one_wrong_output():
    rng = np.random.default_rng(0)
    T, k, H = 64, 8, 256
    y = rng.standard_normal((T * k, H)).astype(np.float32)
    s2r = rng.permutation(T * k).astype(np.int32)
    w = rng.random((T, k)).astype(np.float32)
    y[s2r[3 * k + 1], :] = -y[s2r[3 * k], :] * (w[3, 0] / w[3, 1])      # cancellation in token 3
    got = _reduce_like_the_kernel(y, s2r, w)
    assert_reduce_elementwise(got, y, s2r, w)
    bad = got.copy()
    bad[7, 9] += 2 * bf16_ulp(bad[7, 9])
    with pytest.raises(AssertionError):
        assert_reduce_elementwise(bad, y, s2r, w)
    nan = got.copy()
    nan[1, 1] = np.nan
    with pytest.raises(AssertionError):
        assert_reduce_elementwise(nan, y, s2r, w)


def test_every_expert_check_catches_a_wrong_expert():
    rng = np.random.default_rng(1)
    E, K, F, H = 6, 64, 128, 64
    counts = np.array([0, 300, 3, 0, 140, 1])
    offsets = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    S = int(offsets[-1])
    tok = rng.integers(0, 100, S)
    A_all = moe.bf16_round(rng.standard_normal((100, K)))
    W13 = [nvfp4.quantize((rng.standard_normal((2 * F, K)) * 0.02).astype(np.float32)) for _ in range(E)]
    W2 = [nvfp4.quantize((rng.standard_normal((H, F)) * 0.02).astype(np.float32)) for _ in range(E)]
    deq13 = lambda e, idx: nvfp4.dequantize(W13[e][0][idx], W13[e][1][idx], W13[e][2])
    deq2 = lambda e, idx: nvfp4.dequantize(W2[e][0][idx], W2[e][1][idx], W2[e][2])
    h = moe.bf16_round(moe.grouped_gemm(A_all[tok], offsets, lambda e: nvfp4.dequantize(*W13[e]), "swiglu"))
    y = moe.grouped_gemm(h, offsets, lambda e: nvfp4.dequantize(*W2[e])).astype(np.float32)
    args = (offsets, tok, A_all, h.astype(np.float32), y, lambda rows: h[rows], deq13, deq2, F, H, moe.bf16_round)
    assert check_every_expert(*args, tol_h=1e-3) == 4
    y_bad = y.copy()
    y_bad[offsets[4]:offsets[5]] = moe.grouped_gemm(h, offsets, lambda e: nvfp4.dequantize(*W2[1]))[offsets[4]:offsets[5]]
    with pytest.raises(AssertionError):
        check_every_expert(*args[:4], y_bad, *args[5:], tol_h=1e-3)
    h_bad = h.astype(np.float32).copy()
    h_bad[offsets[1] + 255] *= 1.01        # the last row of a 64-row block of a large expert
    with pytest.raises(AssertionError):
        check_every_expert(*args[:3], h_bad, *args[4:], tol_h=1e-3)
