"""The no-allocation quantize entry point against the workspace entry point, through the C ABI.

nvfp4_quantize_noalloc keeps the amax pass's partial maxima in a 64 KiB scratch array that the
library holds on each GPU; every call reuses it. Two calls in a row (the first filling the
scratch exactly, the second smaller, with NaN/Inf/zero groups) must each give the same bytes
as nvfp4_quantize with a caller workspace.
"""
import ctypes

import numpy as np
import pytest
import torch

from nvfp4_block_scaled_moe_amd import _lib, inputs, ops
from tests.gpu_util import say

pytestmark = pytest.mark.gpu
DEV = "cuda"


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _noalloc(x):
    """Quantize [B, R, C] with nvfp4_quantize_noalloc into outputs prefilled with 0xAB/NaN."""
    B, R, C = x.shape
    packed = torch.full((B, R, C // 2), 0xAB, dtype=torch.uint8, device=DEV)
    scales = torch.full((B, R, C // 16), 0xAB, dtype=torch.uint8, device=DEV)
    g = torch.full((B,), float("nan"), dtype=torch.float32, device=DEV)
    lib = _lib.load()
    st = lib.nvfp4_quantize_noalloc(ctypes.c_void_p(x.data_ptr()), _lib.BF16 if x.dtype == torch.bfloat16 else _lib.F32,
                                    B, R, C, None, None, _lib.LAYOUT_ROW_MAJOR, ctypes.c_void_p(packed.data_ptr()),
                                    ctypes.c_void_p(scales.data_ptr()), ctypes.c_void_p(g.data_ptr()),
                                    ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    _lib.check("nvfp4_quantize_noalloc", st)
    return packed, scales, g


def test_noalloc_quantize_matches_workspace_call_on_two_calls():
    lib = _lib.load()
    cases = [(16, 4096, 4096, torch.bfloat16), (3, 37, 96, torch.float32)]
    assert lib.nvfp4_quantize_workspace_size(*cases[0][:3]) == 65536         # the scratch limit
    for i, (B, R, C, dt) in enumerate(cases):
        say("quantize_noalloc call", i, B, R, C, dt)
        x = torch.stack([inputs.random_fp32((R, C), 7000 + 31 * i + b, std=0.02 * (b + 1), device=DEV)
                         for b in range(B)]).to(dt)
        if i == 1:
            x[0, 2, 0:16] = 0.0
            x[1, 5, 17] = float("nan")
            x[2, 30, 40] = float("inf")
        got = _noalloc(x)
        torch.cuda.synchronize()
        want = ops.nvfp4_quantize(x)
        torch.cuda.synchronize()
        for a, b, name in zip(got, want, ("packed", "scales", "g")):
            assert torch.equal(a.view(torch.uint8) if a.dtype != torch.uint8 else a,
                               b.view(torch.uint8) if b.dtype != torch.uint8 else b), name
        assert np.isfinite(got[2].cpu().numpy()).all()
        del x, got, want
