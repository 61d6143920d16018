"""GPU parity of the whole MoE layer (route -> up/gate + SwiGLU -> down -> reduce).

The tiny workload is checked end to end against the oracle's layer. The full-size
workloads run exactly the sequence of calls the benchmark times; the oracle checks routing
and permutation in full, the activation and h codes in full (W4A4), the weight quantization
on the largest, median and smallest active expert, both GEMMs on every active expert (fed
the GPU's inputs to each stage; rows at both edges of every 64-row block and 4 columns of
every 64-column block), and the reduce in full, element by element.
"""
import numpy as np
import pytest
import torch

from nvfp4_block_scaled_moe_amd import inputs, layer, ops
from oracle import moe as omoe
from oracle import nvfp4 as onv
from tests.gpu_util import assert_finite, assert_reduce_elementwise, check_every_expert, np_, rel_fro, say

pytestmark = pytest.mark.gpu
DEV = "cuda"


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _oracle_experts(w):
    return (lambda e: (np_(w.w13_packed[e]), np_(w.w13_scales[e]), np_(w.w13_g[e:e + 1])[0]),
            lambda e: (np_(w.w2_packed[e]), np_(w.w2_scales[e]), np_(w.w2_g[e:e + 1])[0]))


@pytest.mark.parametrize("mode", [ops.W4A16, ops.W4A4])
def test_tiny_layer_end_to_end(mode):
    wl = inputs.WORKLOADS["tiny"]
    say("tiny layer", mode)
    w = layer.quantize_experts(wl, DEV)
    x = inputs.activations_bf16(wl)
    lg = inputs.router_logits(wl)
    out, st = layer.moe_forward(x.to(DEV), lg.to(DEV), wl.k, w, mode=mode, keep=True)
    torch.cuda.synchronize()
    w13, w2 = _oracle_experts(w)
    for e in range(wl.E):   # weight quantization bit-exact
        po, so, go = onv.quantize(inputs.expert_weight_fp32(wl, "w13", e, DEV).cpu().numpy())
        assert np.array_equal(w13(e)[0], po) and np.array_equal(w13(e)[1], so) and w13(e)[2] == go
    want, ost = omoe.moe_layer(x.float().numpy(), lg.numpy(), wl.k, w13, w2,
                               mode="w4a16" if mode == ops.W4A16 else "w4a4", return_stages=True)
    got = np_(out)
    assert_finite(got)
    assert np.array_equal(np_(st["topk_ids"]), ost["ids"])
    assert np.array_equal(np_(st["sorted_slot"]), ost["perm"]["sorted_slot"])
    tol = 1e-3 if mode == ops.W4A16 else 2e-2
    r = rel_fro(got, want)
    say("tiny layer rel err", r)
    assert r <= tol
    if mode == ops.W4A4:
        assert np.array_equal(np_(st["xq"]), ost["xq"][0]) and np.array_equal(np_(st["xs"]), ost["xq"][1])


@pytest.mark.parametrize("path", ["stream", "mfma"])
def test_tiny_w4a4_layer_nan_token_stays_local(path, monkeypatch):
    """A NaN in one token's activations: its NVFP4 group gets a NaN scale, so every h and Y row
    of that token's slots is NaN. h's global scale comes from the finite amax, so no other
    token is touched: exactly the oracle's NaN pattern (one output row), the rest within the
    W4A4 tolerance of the oracle, on both GEMM paths."""
    say("tiny w4a4 layer, NaN token", path)
    monkeypatch.setenv("NVFP4MOE_FORCE_PATH", path)
    wl = inputs.WORKLOADS["tiny"]
    w = layer.quantize_experts(wl, DEV)
    x = inputs.activations_bf16(wl).clone()
    x[5, 40] = float("nan")
    lg = inputs.router_logits(wl)
    out, st = layer.moe_forward(x.to(DEV), lg.to(DEV), wl.k, w, mode=ops.W4A4, keep=True)
    torch.cuda.synchronize()
    assert np.isfinite(np_(st["h_amax"])).all() and np.isfinite(np_(st["hg"])).all()
    w13, w2 = _oracle_experts(w)
    want = omoe.moe_layer(x.float().numpy(), lg.numpy(), wl.k, w13, w2, mode="w4a4")
    got = np_(out)
    nan_rows = np.nonzero(np.isnan(want).any(axis=1))[0]
    assert list(nan_rows) == [5] and np.isnan(want[5]).all()
    assert np.array_equal(np.isnan(got), np.isnan(want))
    keep = np.arange(wl.T) != 5
    assert rel_fro(got[keep], want[keep]) <= 2e-2


def _sample_experts(offsets, n=3):
    counts = np.diff(offsets)
    act = np.nonzero(counts)[0]
    order = act[np.argsort(counts[act], kind="stable")]
    picks = {int(order[-1]), int(order[len(order) // 2]), int(order[0])}
    return sorted(picks)[:n]


def _dequant_rows(packed, scales, g):
    """deq(e, idx): float64 rows idx of expert e's NVFP4 matrix, dequantized by the oracle
    from the GPU's codes (only those rows leave the device)."""
    def deq(e, idx):
        ix = torch.from_numpy(np.asarray(idx, dtype=np.int64)).to(packed.device)
        return onv.dequantize(np_(packed[e][ix]), np_(scales[e][ix]), np_(g[e:e + 1])[0])
    return deq


def _check_full_size(wl, T, mode, fp8=False):
    say("full-size layer", wl.name, T, mode)
    w = layer.quantize_experts(wl, DEV)
    x = inputs.activations_bf16(wl, T).to(DEV)
    lg = inputs.router_logits(wl, T)
    out, st = layer.moe_forward(x, lg.to(DEV), wl.k, w, mode=mode, fp8_acts=fp8, keep=True)
    torch.cuda.synchronize()
    # routing and permutation: full, bit-exact
    ids, rw = omoe.route(lg.numpy(), wl.k)
    perm = omoe.permute(ids, wl.E)
    assert np.array_equal(np_(st["topk_ids"]), ids)
    np.testing.assert_allclose(np_(st["topk_w"]), rw, rtol=1e-6, atol=0)
    for key, ref in [("expert_offsets", perm["offsets"]), ("sorted_slot", perm["sorted_slot"]),
                     ("slot_to_row", perm["slot_to_row"])]:
        assert np.array_equal(np_(st[key]), ref), key
    offsets = perm["offsets"]
    xs = np_(st["x_fp8"] if fp8 else x).astype(np.float64)
    if fp8:
        assert np.array_equal(xs, omoe.fp8_roundtrip_bf16(np_(x)))
    if mode == ops.W4A4:
        xq = onv.quantize(xs.astype(np.float32))
        assert np.array_equal(np_(st["xq"]), xq[0]) and np.array_equal(np_(st["xs"]), xq[1])
        A_all = onv.dequantize(*xq)
    else:
        A_all = xs
    tok = perm["sorted_slot"] // wl.k
    h = np_(st["h"])
    y = np_(st["y"])
    assert_finite(h, y)
    if mode == ops.W4A4:
        hq = (np_(st["hq"]), np_(st["hs"]), np_(st["hg"])[0])
        hq_o = onv.quantize(h.astype(np.float32), g=None)
        assert np.array_equal(hq[0], hq_o[0]) and np.array_equal(hq[1], hq_o[1])   # same fp32 h in
        assert hq[2] == hq_o[2]
        h_in_rows = lambda rows: onv.dequantize(hq[0][rows], hq[1][rows], hq[2])
    else:
        h_in_rows = lambda rows: h[rows].astype(np.float64)
    # weight quantization bit-exact on the largest, median and smallest active expert
    for e in _sample_experts(offsets):
        po, so, go = onv.quantize(inputs.expert_weight_fp32(wl, "w13", e, DEV).cpu().numpy())
        assert np.array_equal(np_(w.w13_packed[e]), po) and np.array_equal(np_(w.w13_scales[e]), so)
        assert np_(w.w13_g[e:e + 1])[0] == go
    # both GEMMs on every active expert (every m-tile and weight-row tile sampled)
    check_every_expert(offsets, tok, A_all, h, y, h_in_rows, _dequant_rows(w.w13_packed, w.w13_scales, w.w13_g),
                       _dequant_rows(w.w2_packed, w.w2_scales, w.w2_g), wl.F, wl.H,
                       omoe.bf16_round if mode == ops.W4A16 else (lambda v: v),
                       tol_h=1e-3 if mode == ops.W4A16 else 1e-5, seed=T)
    got = np_(out)
    assert_finite(got)
    assert_reduce_elementwise(got, y, perm["slot_to_row"], np_(st["topk_w"]))


@pytest.mark.parametrize("T", [1, 64, 512])
def test_decode_layer_full_size(T):
    _check_full_size(inputs.WORKLOADS["decode"], T, ops.W4A16)


@pytest.mark.parametrize("T", [1, 64])
def test_many_small_layer_full_size(T):
    _check_full_size(inputs.WORKLOADS["many_small"], T, ops.W4A16, fp8=True)


def test_prefill_layer_full_size():
    _check_full_size(inputs.WORKLOADS["prefill"], 8192, ops.W4A4)


def test_prefill_layer_fp4_staging_bit_identical(monkeypatch):
    """The prefill layer (W4A4, large-M path) with the GEMMs decoding the NVFP4 activation rows
    in their staging gives the same bits as with the f16 copies of the activation prep."""
    wl = inputs.WORKLOADS["prefill"]
    say("prefill layer, fp4 staging")
    w = layer.quantize_experts(wl, DEV)
    x = inputs.activations_bf16(wl).to(DEV)
    lg = inputs.router_logits(wl).to(DEV)
    monkeypatch.delenv("NVFP4MOE_LARGE_A4", raising=False)
    want = layer.moe_forward(x, lg, wl.k, w, mode=ops.W4A4)
    monkeypatch.setenv("NVFP4MOE_LARGE_A4", "1")
    got = layer.moe_forward(x, lg, wl.k, w, mode=ops.W4A4)
    torch.cuda.synchronize()
    assert torch.equal(got, want)


@pytest.mark.parametrize("mode", [ops.W4A16, ops.W4A4])
def test_dense_gemm_full_size(mode):
    wl = inputs.WORKLOADS["dense"]
    say("dense", mode)
    wf = inputs.expert_weight_fp32(wl, "dense", 0, DEV)
    wp, ws, wg = ops.nvfp4_quantize(wf.unsqueeze(0))
    x = inputs.activations_bf16(wl).to(DEV)
    one = lambda v: torch.tensor(v, dtype=torch.int32, device=DEV)
    kw = dict(out_dtype=torch.float32)
    if mode == ops.W4A4:
        aq, as_, ag = ops.nvfp4_quantize(x)
        a = aq
        kw.update(a_scales=as_, a_g=ag)
    else:
        a = x
    wt = ops.nvfp4_weights_tile(wp, ws, wg)
    out = ops.moe_grouped_gemm_nvfp4(mode, ops.EPI_NONE, a, wt, one([0, wl.T]), one([0]), one([1]), **kw)
    torch.cuda.synchronize()
    po, so, go = onv.quantize(wf.cpu().numpy())
    assert np.array_equal(np_(wp[0]), po) and np.array_equal(np_(ws[0]), so)
    A = np_(x).astype(np.float64) if mode == ops.W4A16 else onv.dequantize(np_(aq), np_(as_), np_(ag)[0])
    want = A @ onv.dequantize(po, so, go).T
    got = np_(out)
    assert_finite(got)
    r = rel_fro(got, want)
    say("dense rel err", r)
    assert r < 1e-5
