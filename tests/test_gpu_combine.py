"""The fused down GEMM + weighted unpermute-reduce (the combine calls) against the two-launch
path: the combine's bf16 output must be bit-identical to the down GEMM writing float32 Y
followed by moe_unpermute_reduce, on both NVFP4 kernel paths (W4A16 and W4A4), with split K
(where the reduce runs as a second kernel of the call), in MXFP4, and for whole layers at the
tiny, decode and prefill sizes; the two-launch result is itself checked element by element
against the oracle's reduce of the same Y.
"""
import numpy as np
import pytest
import torch

from nvfp4_block_scaled_moe_amd import inputs, layer, ops
from tests.gpu_util import assert_finite, assert_reduce_elementwise, np_, say

pytestmark = pytest.mark.gpu
DEV = "cuda"


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _routing(T, E, k, seed):
    lg = inputs.random_fp32((T, E), seed).to(DEV)
    return ops.moe_route_permute(lg, k)


def _two_launch(mode, a, w, r, kw):
    common = dict(expert_offsets=r["expert_offsets"], active_experts=r["active_experts"], n_active=r["n_active"])
    y = ops.moe_grouped_gemm_nvfp4(mode, ops.EPI_NONE, a, w, out_dtype=torch.float32, **common, **kw)
    return y, ops.moe_unpermute_reduce(y, r["slot_to_row"], r["topk_w"])


COMBINE_CASES = [
    # T, E, k, H (= Nw of the down GEMM), F (= K)
    (37, 5, 3, 256, 512),
    (16, 8, 1, 512, 256),
    (200, 16, 8, 768, 1024),
    (64, 64, 22, 256, 256),
]


@pytest.mark.parametrize("path", ["stream", "mfma"])
@pytest.mark.parametrize("mode", [ops.W4A16, ops.W4A4])
@pytest.mark.parametrize("T,E,k,H,F", COMBINE_CASES)
def test_combine_equals_gemm_then_reduce(path, mode, T, E, k, H, F, monkeypatch):
    say("combine", path, mode, T, E, k, H, F)
    monkeypatch.setenv("NVFP4MOE_FORCE_PATH", path)
    r = _routing(T, E, k, 1000 + T + k)
    wf = torch.stack([inputs.random_fp32((H, F), 77 + e, std=0.02) for e in range(E)]).to(DEV)
    w = ops.nvfp4_quantize(wf, tiled=True)
    a = inputs.random_fp32((T * k, F), 5 + T).to(torch.bfloat16).to(DEV)
    kw = {}
    if mode == ops.W4A4:
        a, s_, g_ = ops.nvfp4_quantize(a)
        kw = dict(a_scales=s_, a_g=g_)
    y, want = _two_launch(mode, a, w, r, kw)
    got = ops.moe_grouped_gemm_nvfp4_combine(mode, a, w, r["expert_offsets"], r["active_experts"], r["n_active"],
                                             r["sorted_slot"], r["slot_to_row"], r["topk_w"], **kw)
    torch.cuda.synchronize()
    assert torch.equal(got, want)
    assert_finite(np_(got))
    assert_reduce_elementwise(np_(got), np_(y), np_(r["slot_to_row"]), np_(r["topk_w"]))
    again = ops.moe_grouped_gemm_nvfp4_combine(mode, a, w, r["expert_offsets"], r["active_experts"],
                                               r["n_active"], r["sorted_slot"], r["slot_to_row"], r["topk_w"], **kw)
    torch.cuda.synchronize()
    assert torch.equal(again, got)


@pytest.mark.parametrize("path,env", [("stream", "NVFP4MOE_STREAM_KSPLIT"), ("mfma", "NVFP4MOE_LARGE_KSPLIT")])
def test_combine_with_split_k(path, env, monkeypatch):
    """A call that splits K writes Y through the split-K reduce and runs the weighted reduce as
    a second kernel: the same bits."""
    say("combine split-k", path)
    monkeypatch.setenv("NVFP4MOE_FORCE_PATH", path)
    monkeypatch.setenv(env, "2")
    T, E, k, H, F = 40, 6, 4, 256, 2048
    r = _routing(T, E, k, 31)
    w = ops.nvfp4_quantize(torch.stack([inputs.random_fp32((H, F), 90 + e, std=0.02) for e in range(E)]).to(DEV),
                           tiled=True)
    a = inputs.random_fp32((T * k, F), 32).to(torch.bfloat16).to(DEV)
    _, want = _two_launch(ops.W4A16, a, w, r, {})
    got = ops.moe_grouped_gemm_nvfp4_combine(ops.W4A16, a, w, r["expert_offsets"], r["active_experts"],
                                             r["n_active"], r["sorted_slot"], r["slot_to_row"], r["topk_w"])
    torch.cuda.synchronize()
    assert torch.equal(got, want)


@pytest.mark.parametrize("T,E,k,H,F", [(37, 5, 3, 256, 512), (300, 8, 2, 512, 256), (64, 64, 8, 256, 256)])
def test_mxfp4_combine_equals_gemm_then_reduce(T, E, k, H, F):
    say("mxfp4 combine", T, E, k, H, F)
    r = _routing(T, E, k, 2000 + T)
    wp, ws_ = [], []
    for e in range(E):
        p, s = ops.mxfp4_quantize(inputs.random_fp32((H, F), 300 + e, std=0.02).to(DEV))
        wp.append(p)
        ws_.append(s)
    w = ops.mxfp4_weights_tile(torch.stack(wp), torch.stack(ws_))
    a, a_s = ops.mxfp4_quantize(inputs.random_fp32((T * k, F), 9).to(DEV))
    common = dict(expert_offsets=r["expert_offsets"], active_experts=r["active_experts"], n_active=r["n_active"])
    y = ops.moe_grouped_gemm_mxfp4(ops.EPI_NONE, a, a_s, w, out_dtype=torch.float32, **common)
    want = ops.moe_unpermute_reduce(y, r["slot_to_row"], r["topk_w"])
    got = ops.moe_grouped_gemm_mxfp4_combine(a, a_s, w, r["expert_offsets"], r["active_experts"], r["n_active"],
                                             r["sorted_slot"], r["slot_to_row"], r["topk_w"])
    torch.cuda.synchronize()
    assert torch.equal(got, want)


@pytest.mark.parametrize("name,T,mode", [("tiny", None, ops.W4A16), ("tiny", None, ops.W4A4),
                                         ("decode", 512, ops.W4A16), ("decode", 1, ops.W4A16),
                                         ("many_small", 64, ops.W4A16), ("prefill", 8192, ops.W4A4)])
def test_layer_combine_bit_identical(name, T, mode):
    wl = inputs.WORKLOADS[name]
    say("layer combine", name, T, mode)
    w = layer.quantize_experts(wl, DEV)
    x = inputs.activations_bf16(wl, T).to(DEV)
    lg = inputs.router_logits(wl, T).to(DEV)
    fp8 = wl.act == "fp8"
    want = layer.moe_forward(x, lg, wl.k, w, mode=mode, fp8_acts=fp8)
    got = layer.moe_forward(x, lg, wl.k, w, mode=mode, fp8_acts=fp8, combine=True)
    torch.cuda.synchronize()
    assert torch.equal(got, want)


def test_mxfp4_prefill_layer_combine_bit_identical():
    wl = inputs.WORKLOADS["prefill"]
    say("mxfp4 prefill layer combine")
    w = layer.quantize_experts_mxfp4(wl, DEV)
    x = inputs.activations_bf16(wl).to(DEV)
    lg = inputs.router_logits(wl).to(DEV)
    want = layer.moe_forward_mxfp4(x, lg, wl.k, w)
    got = layer.moe_forward_mxfp4(x, lg, wl.k, w, combine=True)
    torch.cuda.synchronize()
    assert torch.equal(got, want)
