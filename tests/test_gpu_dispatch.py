"""moe_dispatch_w4a16 (routing + the W4A16 preparation of the token rows, one launch for up to
16 tokens) against the separate calls: its routing outputs must be bit-identical to
moe_route_permute's, and the up/gate GEMM on its prepared rows (mode W4A16_PREPARED) bit for
bit the GEMM on the bf16 rows (after act_fp8_e4m3_roundtrip when the FP8 activations are
asked for), whose parity with the oracle the GEMM tests establish. Covered: the one-launch
path (T <= 16, rows up to 8192 columns), its fallbacks (more tokens, longer rows: routing
then separate preparation launches), FP8 activations on both, NaN / Inf / zero rows, and the
whole layer (layer.moe_forward dispatches) against the separate calls.
"""
import numpy as np
import pytest
import torch

from nvfp4_block_scaled_moe_amd import inputs, layer, ops
from tests.gpu_util import np_, say

pytestmark = pytest.mark.gpu
DEV = "cuda"


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _bits(t):
    """Integer view of a float tensor: bitwise comparison (NaN payloads included)."""
    return t.contiguous().view(torch.int32 if t.dtype == torch.float32 else torch.int16)


DISPATCH_CASES = [
    # T, E, k, H, fp8
    (1, 256, 8, 6144, 0),      # decode, one token
    (1, 512, 22, 4096, 1),     # many-small, one token, FP8 activations
    (16, 256, 8, 6144, 0),     # the largest one-launch batch
    (16, 512, 22, 4096, 1),
    (3, 1000, 17, 256, 0),     # odd E and k, short rows
    (5, 64, 4, 8192, 1),       # the longest row of the one-launch path
    (2, 64, 4, 8224, 0),       # longer rows: routing in one launch, rows prepared after it
    (2, 64, 4, 8224, 1),
    (17, 256, 8, 2048, 0),     # more tokens: separate routing launches, then the rows
    (64, 512, 22, 4096, 1),
    (7, 40, 3, 160, 0),        # H % 128 != 0 (zero-padded chunk)
    (16, 1024, 64, 64, 1),     # the most slots (1024) and experts of the one-launch path, short rows
    (4, 32, 2, 32, 0),         # the shortest rows
]


@pytest.mark.parametrize("T,E,k,H,fp8", DISPATCH_CASES)
def test_dispatch_equals_route_then_gemm(T, E, k, H, fp8):
    say("dispatch", T, E, k, H, fp8)
    lg = inputs.random_fp32((T, E), 300 + T + E).to(DEV)
    x = inputs.random_fp32((T, H), 400 + T + H).to(torch.bfloat16)
    if T >= 3:
        x[1, 5] = float("nan")        # a NaN element: its row's outputs NaN, the others finite
        x[2] = 0.0                    # an all-zero row (exponent 0)
        x[2, 7] = float("inf")        # ... with one Inf
    x = x.to(DEV)
    d = ops.moe_dispatch_w4a16(lg, x, k, fp8_act=bool(fp8))
    r = ops.moe_route_permute(lg, k)
    torch.cuda.synchronize()
    for key in ("topk_ids", "expert_offsets", "sorted_slot", "slot_to_row", "n_active"):
        assert torch.equal(d[key], r[key]), key
    na = int(r["n_active"].item())
    assert torch.equal(d["active_experts"][:na], r["active_experts"][:na])
    assert torch.equal(_bits(d["topk_w"]), _bits(r["topk_w"]))
    # the up/gate GEMM (SwiGLU, small weights) on the prepared rows against the bf16 rows
    Nw = 64
    wf = torch.stack([inputs.random_fp32((Nw, H), 77 + e, std=0.02) for e in range(E)]).to(DEV)
    w = ops.nvfp4_quantize(wf, tiled=True)
    xx = ops.act_fp8_e4m3_roundtrip(x) if fp8 else x
    common = dict(expert_offsets=r["expert_offsets"], active_experts=r["active_experts"], n_active=r["n_active"],
                  gather_index=r["sorted_slot"], gather_div=k, rows=T * k)
    for odt in (torch.float32, torch.bfloat16):
        want = ops.moe_grouped_gemm_nvfp4(ops.W4A16, ops.EPI_SWIGLU, xx, w, out_dtype=odt, **common)
        got = ops.moe_grouped_gemm_nvfp4(ops.W4A16_PREPARED, ops.EPI_SWIGLU, d["x_prep"], w, a_rows=T,
                                         out_dtype=odt, **common)
        torch.cuda.synchronize()
        assert torch.equal(_bits(got), _bits(want))
    if T >= 3:
        o = np_(got.float())
        bad = np.isin(np_(r["sorted_slot"]) // k, [1, 2])
        assert np.isnan(o[bad]).any() and np.isfinite(o[~bad]).all()


@pytest.mark.parametrize("path", ["stream", "mfma"])
def test_prepared_rows_on_both_gemm_paths(path, monkeypatch):
    """The prepared rows feed either GEMM kernel (the MFMA path then builds its m-tile list in
    a launch of its own)."""
    say("prepared rows", path)
    monkeypatch.setenv("NVFP4MOE_FORCE_PATH", path)
    T, E, k, H = 12, 4, 2, 1024
    lg = inputs.random_fp32((T, E), 5).to(DEV)
    x = inputs.random_fp32((T, H), 6).to(torch.bfloat16).to(DEV)
    d = ops.moe_dispatch_w4a16(lg, x, k)
    wf = torch.stack([inputs.random_fp32((256, H), 7 + e, std=0.02) for e in range(E)]).to(DEV)
    w = ops.nvfp4_quantize(wf, tiled=True)
    common = dict(expert_offsets=d["expert_offsets"], active_experts=d["active_experts"], n_active=d["n_active"],
                  gather_index=d["sorted_slot"], gather_div=k, rows=T * k, out_dtype=torch.float32)
    for epi in (ops.EPI_NONE, ops.EPI_SWIGLU):
        want = ops.moe_grouped_gemm_nvfp4(ops.W4A16, epi, x, w, **common)
        got = ops.moe_grouped_gemm_nvfp4(ops.W4A16_PREPARED, epi, d["x_prep"], w, a_rows=T, **common)
        assert ops.last_dispatch() == (ops.PATH_STREAM if path == "stream" else ops.PATH_MFMA)
        torch.cuda.synchronize()
        assert torch.equal(_bits(got), _bits(want))


@pytest.mark.parametrize("ksplit", ["2", "3"])
def test_prepared_rows_with_split_k(ksplit, monkeypatch):
    """Prepared rows under the small-M kernel's K split (a tiny grid: one token, few experts)."""
    say("prepared rows split-k", ksplit)
    monkeypatch.setenv("NVFP4MOE_FORCE_PATH", "stream")
    monkeypatch.setenv("NVFP4MOE_STREAM_KSPLIT", ksplit)
    T, E, k, H = 1, 8, 2, 3072
    lg = inputs.random_fp32((T, E), 11).to(DEV)
    x = inputs.random_fp32((T, H), 12).to(torch.bfloat16).to(DEV)
    d = ops.moe_dispatch_w4a16(lg, x, k)
    wf = torch.stack([inputs.random_fp32((128, H), 13 + e, std=0.02) for e in range(E)]).to(DEV)
    w = ops.nvfp4_quantize(wf, tiled=True)
    common = dict(expert_offsets=d["expert_offsets"], active_experts=d["active_experts"], n_active=d["n_active"],
                  gather_index=d["sorted_slot"], gather_div=k, rows=T * k, out_dtype=torch.float32)
    want = ops.moe_grouped_gemm_nvfp4(ops.W4A16, ops.EPI_SWIGLU, x, w, **common)
    got = ops.moe_grouped_gemm_nvfp4(ops.W4A16_PREPARED, ops.EPI_SWIGLU, d["x_prep"], w, a_rows=T, **common)
    torch.cuda.synchronize()
    assert torch.equal(_bits(got), _bits(want))


@pytest.mark.parametrize("wl_name,T", [("tiny", 16), ("decode", 1), ("decode", 16), ("many_small", 1),
                                       ("many_small", 4)])
def test_layer_dispatch_equals_separate_calls(wl_name, T):
    """layer.moe_forward (dispatch + prepared GEMM) against the same layer written with the
    separate calls (FP8 round trip, moe_route_permute, the GEMM's own row preparation)."""
    say("layer dispatch", wl_name, T)
    wl = inputs.WORKLOADS[wl_name]
    w = layer.quantize_experts(wl, DEV)
    x = inputs.activations_bf16(wl, T).to(DEV)
    lg = inputs.router_logits(wl, T).to(DEV)
    fp8 = wl.act == "fp8"
    got = layer.moe_forward(x, lg, wl.k, w, fp8_acts=fp8)
    xx = ops.act_fp8_e4m3_roundtrip(x) if fp8 else x
    r = ops.moe_route_permute(lg, wl.k)
    common = dict(expert_offsets=r["expert_offsets"], active_experts=r["active_experts"], n_active=r["n_active"])
    S = T * wl.k
    h = ops.moe_grouped_gemm_nvfp4(ops.W4A16, ops.EPI_SWIGLU, xx, w.w13_t, gather_index=r["sorted_slot"],
                                   gather_div=wl.k, rows=S, out_dtype=torch.bfloat16, **common)
    y = ops.moe_grouped_gemm_nvfp4(ops.W4A16, ops.EPI_NONE, h, w.w2_t, rows=S, out_dtype=torch.float32, **common)
    want = ops.moe_unpermute_reduce(y, r["slot_to_row"], r["topk_w"])
    torch.cuda.synchronize()
    assert torch.equal(_bits(got), _bits(want))


def test_dispatch_argument_errors():
    lg = torch.zeros((2, 8), device=DEV)
    x = torch.zeros((2, 48), dtype=torch.bfloat16, device=DEV)   # H % 32 != 0
    with pytest.raises(ops._lib.NVFP4MoEError):
        ops.moe_dispatch_w4a16(lg, x, 2)
    with pytest.raises(ValueError):
        ops.moe_grouped_gemm_nvfp4(ops.W4A16_PREPARED, ops.EPI_NONE, torch.zeros(16, dtype=torch.uint8, device=DEV),
                                   ops.nvfp4_quantize(torch.zeros((1, 32, 64), device=DEV), tiled=True),
                                   torch.tensor([0, 2], dtype=torch.int32, device=DEV),
                                   torch.zeros(1, dtype=torch.int32, device=DEV),
                                   torch.ones(1, dtype=torch.int32, device=DEV))
