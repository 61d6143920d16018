"""GPU parity of the MXFP4 variant (group-32 UE8M0 scales) against the MXFP4 oracle.

The quantizer's codes and scales and the tiled scale storage must match bit for bit; the
W4A4 grouped GEMM on the scaled FP4 matrix cores must match the float64 oracle fed the same
dequantized operands (summation order is the only difference, < 1e-5 relative Frobenius in
float32 output, and within the W4A4 bound in bf16).
"""
import numpy as np
import pytest
import torch

from nvfp4_block_scaled_moe_amd import _lib, inputs, ops
from oracle import moe as omoe
from oracle import mxfp4 as omx
from tests.gpu_util import assert_finite, assert_reduce_elementwise, check_every_expert, np_, rel_fro, say

pytestmark = pytest.mark.gpu
DEV = "cuda"
W4A4_TOL = 2e-2


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    torch.cuda.init()


# ------------------------------------------------------------------ quantize
def _special(R, C, seed):
    x = inputs.random_fp32((R, C), seed, std=1.0)
    x[0, :32] = 0.0
    x[0, 5] = -0.0
    if R > 1 and C >= 128:
        x[1, 32:64] *= 2.0 ** -130            # below the smallest scale: e clamps at -127
        x[1, 64:96] *= 2.0 ** 100             # large exponents
        x[1, 100] = float("nan")
        x[1, 33] = float("inf")
        x[1, 96:128] = 7.0                    # saturation at 6 * 2^0
        x[1, 97] = 2.5                        # a tie (2.5 -> 2) in the same group
    return x


@pytest.mark.parametrize("R,C,dt", [(4, 128, torch.float32), (33, 96, torch.float32), (64, 2048, torch.float32),
                                    (5, 4096, torch.bfloat16), (2, 128, torch.bfloat16)])
def test_mxfp4_quantize_bit_exact(R, C, dt):
    say("mx quantize", R, C, dt)
    x = _special(R, C, R + C).to(dt)
    p, s = ops.mxfp4_quantize(x.to(DEV))
    torch.cuda.synchronize()
    wp, ws = omx.quantize(x.float().numpy())
    assert np.array_equal(np_(p), wp)
    assert np.array_equal(np_(s), ws)


def test_mxfp4_quantize_codes_at_every_rounding_threshold():
    """E2M1 codes at unit scale on both sides of every E2M1 rounding midpoint (0.25, 0.75,
    1.25, 1.75, 2.5, 3.5, 5): the 2048 float32 values below and above each midpoint, both
    signs, plus zeros, subnormals and values up to 8 that saturate at 6. Each group of 32 holds
    a 4.0, so its scale exponent is 0 and every other code is E2M1 of the value itself."""
    mids = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0], np.float32)
    bits = mids.view(np.uint32).astype(np.int64)[:, None] + np.arange(-2048, 2049, dtype=np.int64)[None, :]
    vals = bits.astype(np.uint32).view(np.float32).ravel()
    extra = np.array([0.0, -0.0, 1.4e-45, -1.4e-45, 1e-40, -1e-40, 5.999, 6.0, 6.5, 7.0, 7.999], np.float32)
    vals = np.concatenate([vals, -vals, extra, -extra])
    groups = -(-vals.size // 31)
    groups = -(-groups // 64) * 64                      # 64 groups (2048 columns) per row
    vals = np.concatenate([vals, np.zeros(groups * 31 - vals.size, np.float32)]).reshape(groups, 31)
    x = np.concatenate([np.full((groups, 1), 4.0, np.float32), vals], axis=1).reshape(-1, 2048)
    say("mx quantize thresholds", x.shape)
    p, s = ops.mxfp4_quantize(torch.from_numpy(x).to(DEV))
    torch.cuda.synchronize()
    wp, ws = omx.quantize(x)
    assert np.all(ws == 127)
    assert np.array_equal(np_(s), ws)
    assert np.array_equal(np_(p), wp)


# ------------------------------------------------------------------ tiling
def _mx_tile_reference(packed, scales):
    """Index-by-index transcription of the MX scale tiles (include/nvfp4moe.h)."""
    B, R, Ch = packed.shape
    C = 2 * Ch
    nch, nwin = -(-C // 128), -(-C // 2048)
    sc = np.zeros((B, R // 16, nwin, 64, 16), np.uint8)
    for b in range(B):
        for row in range(R):
            rb, r = divmod(row, 16)
            for g in range(4):
                for w in range(nwin):
                    for u in range(16):
                        k0 = 128 * (16 * w + u) + 32 * g
                        if k0 < C:
                            sc[b, rb, w, 16 * g + r, u] = scales[b, row, k0 // 32]
    return sc.reshape(B, -1)


@pytest.mark.parametrize("B,R,C", [(1, 16, 32), (2, 48, 160), (1, 32, 2176), (2, 16, 4096)])
def test_mxfp4_weights_tile_bit_exact(B, R, C):
    say("mx tile", B, R, C)
    rng = np.random.default_rng(B * 3 + R + C)
    packed = rng.integers(0, 256, size=(B, R, C // 2), dtype=np.uint8)
    scales = rng.integers(0, 256, size=(B, R, C // 32), dtype=np.uint8)
    t = ops.mxfp4_weights_tile(torch.from_numpy(packed).to(DEV), torch.from_numpy(scales).to(DEV))
    nv = ops.nvfp4_weights_tile(torch.from_numpy(packed).to(DEV),
                                torch.zeros((B, R, C // 16), dtype=torch.uint8, device=DEV),
                                torch.ones(B, device=DEV))
    torch.cuda.synchronize()
    assert np.array_equal(np_(t.codes), np_(nv.codes))        # the same code tiles as NVFP4
    assert np.array_equal(np_(t.scales), _mx_tile_reference(packed, scales))


# ------------------------------------------------------------------ grouped GEMM
def _mx_problem(counts, Nw, K, seed, T=None, k=None):
    E = len(counts)
    offsets = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    rows = int(offsets[-1])
    act = [e for e in range(E) if counts[e] > 0]
    active = np.array(act + [-1] * (E - len(act)), np.int32)
    w = torch.stack([inputs.random_fp32((Nw, K), seed + 17 * e, std=0.02) for e in range(E)])
    wp, ws = ops.mxfp4_quantize(w.to(DEV))
    nA = rows if T is None else T
    a = inputs.random_fp32((nA, K), seed + 1).to(torch.bfloat16)
    ap, as_ = ops.mxfp4_quantize(a.to(DEV))
    A = omx.dequantize(np_(ap), np_(as_))
    gidx = None
    if T is not None:
        gidx = np.random.default_rng(seed).integers(0, T * k, size=rows).astype(np.int32)
        A = A[gidx // k]
    return dict(E=E, rows=rows, offsets=offsets, active=active, n_active=np.array([len(act)], np.int32),
                wt=ops.mxfp4_weights_tile(wp, ws), ap=ap, as_=as_, A=A, gidx=gidx, gdiv=k or 1,
                W=[omx.dequantize(np_(wp[e]), np_(ws[e])) for e in range(E)])


def _run(d, epi, out_dtype, want_amax=False):
    t = lambda x: torch.from_numpy(x).to(DEV)
    res = ops.moe_grouped_gemm_mxfp4(epi, d["ap"], d["as_"], d["wt"], t(d["offsets"]), t(d["active"]),
                                     t(d["n_active"]), rows=d["rows"], out_dtype=out_dtype,
                                     gather_index=None if d["gidx"] is None else t(d["gidx"]),
                                     gather_div=d["gdiv"], want_amax=want_amax)
    torch.cuda.synchronize()
    return res


MX_CASES = [
    # counts per expert, Nw, K
    ([150, 0, 40, 270], 512, 640),       # ragged m-tiles, a 0-row expert, K % 128 != 0
    ([128], 256, 2048),                  # one full m-tile, one scale window
    ([300, 7], 256, 4096 + 96),          # two scale windows and a partial one
    ([1, 2, 3, 500], 768, 256),          # three row tiles, tiny experts
    ([513], 256, 7168),                  # the prefill hidden size (partial last window)
]


@pytest.mark.parametrize("counts,Nw,K", MX_CASES)
def test_grouped_gemm_mxfp4(counts, Nw, K):
    say("gemm mxfp4", counts, Nw, K)
    d = _mx_problem(counts, Nw, K, seed=Nw + K)
    for epi in (ops.EPI_NONE, ops.EPI_SWIGLU):
        want = omoe.grouped_gemm(d["A"], d["offsets"], d["W"], "swiglu" if epi else "none")
        got = np_(_run(d, epi, torch.float32))
        assert_finite(got)
        r = rel_fro(got, want)
        assert r < 1e-5, r          # identical operands on both sides: only summation order differs
        got16 = np_(_run(d, epi, torch.bfloat16))
        assert rel_fro(got16, omoe.bf16_round(want)) <= W4A4_TOL


@pytest.mark.parametrize("counts,Nw,K", MX_CASES)
def test_grouped_gemm_mxfp4_split_k(counts, Nw, K, monkeypatch):
    """K forced into 3 slices of whole chunks (slices that start inside a scale window, and a
    window crossed by a slice), summed by the fixed-order split-K reduce."""
    say("gemm mxfp4 split-k", counts, Nw, K)
    monkeypatch.setenv("NVFP4MOE_MX_KSPLIT", "3")
    d = _mx_problem(counts, Nw, K, seed=Nw + K + 1)
    for epi in (ops.EPI_NONE, ops.EPI_SWIGLU):
        want = omoe.grouped_gemm(d["A"], d["offsets"], d["W"], "swiglu" if epi else "none")
        got, amax = _run(d, epi, torch.float32, want_amax=True)
        got = np_(got)
        assert_finite(got)
        assert rel_fro(got, want) < 1e-5
        assert np_(amax)[0] == np.abs(got).max()


def test_dense_mxfp4_gemm_full_size():
    """The dense GEMM M=512, N=2048, K=6144 in MXFP4 (a grid of 32 tiles: K split on its own
    into 7 slices of 7 chunks), full output against the oracle."""
    wl = inputs.WORKLOADS["dense"]
    say("dense mxfp4")
    wp, ws = ops.mxfp4_quantize(inputs.expert_weight_fp32(wl, "dense", 0, DEV).unsqueeze(0))
    x = inputs.activations_bf16(wl).to(DEV)
    ap, as_ = ops.mxfp4_quantize(x)
    one = lambda v: torch.tensor(v, dtype=torch.int32, device=DEV)
    out = ops.moe_grouped_gemm_mxfp4(ops.EPI_NONE, ap, as_, ops.mxfp4_weights_tile(wp, ws), one([0, wl.T]),
                                     one([0]), one([1]), out_dtype=torch.float32)
    torch.cuda.synchronize()
    want = omx.dequantize(np_(ap), np_(as_)) @ omx.dequantize(np_(wp[0]), np_(ws[0])).T
    got = np_(out)
    assert_finite(got)
    r = rel_fro(got, want)
    say("dense mxfp4 rel err", r)
    assert r < 1e-5


@pytest.mark.parametrize("group,ksplit", [("3", "1"), ("2", "3"), ("64", "1"), ("1", "1")])
def test_grouped_gemm_mxfp4_tile_groups(group, ksplit, monkeypatch):
    """The tile order within an expert: m-tiles in groups whose tiles run row-tile-major. Here
    experts hold several groups (the last group shorter, the last m-tile ragged), with and
    without K slices, so every (m-tile, row tile) pair must still be computed exactly once."""
    counts = [1000, 0, 300, 129]         # 8, 0, 3 and 2 m-tiles of 128 rows
    say("gemm mxfp4 tile groups", group, ksplit)
    monkeypatch.setenv("NVFP4MOE_MX_GROUP", group)
    monkeypatch.setenv("NVFP4MOE_MX_KSPLIT", ksplit)
    d = _mx_problem(counts, 768, 640, seed=91)
    for epi in (ops.EPI_NONE, ops.EPI_SWIGLU):
        want = omoe.grouped_gemm(d["A"], d["offsets"], d["W"], "swiglu" if epi else "none")
        got = np_(_run(d, epi, torch.float32))
        assert_finite(got)
        assert rel_fro(got, want) < 1e-5


@pytest.mark.parametrize("counts,Nw,K,T,k", [(c, n, kk, None, None) for c, n, kk in MX_CASES]
                         + [([7, 0, 300, 9], 256, 512, 120, 3)])
def test_swiglu_q_codes_bit_exact(counts, Nw, K, T, k):
    """h quantized to MXFP4 by the up/gate epilogue: codes and scales equal, bit for bit, the
    oracle's MXFP4 quantization of the float32 h of the unquantized call (same arithmetic in
    both epilogues), and that h matches the float64 oracle."""
    say("swiglu_q", counts, Nw, K, T, k)
    d = _mx_problem(counts, Nw, K, seed=Nw + K + 2, T=T, k=k)
    h32 = np_(_run(d, ops.EPI_SWIGLU, torch.float32))
    assert rel_fro(h32, omoe.grouped_gemm(d["A"], d["offsets"], d["W"], "swiglu")) < 1e-5
    t = lambda x: torch.from_numpy(x).to(DEV)
    hp, hs = ops.moe_grouped_gemm_mxfp4_swiglu_q(d["ap"], d["as_"], d["wt"], t(d["offsets"]), t(d["active"]),
                                                 t(d["n_active"]), rows=d["rows"], gather_div=d["gdiv"],
                                                 gather_index=None if d["gidx"] is None else t(d["gidx"]))
    torch.cuda.synchronize()
    qp, qs = omx.quantize(h32.astype(np.float32))
    assert np.array_equal(np_(hp), qp)
    assert np.array_equal(np_(hs), qs)


def test_grouped_gemm_mxfp4_gather_and_amax():
    say("gemm mxfp4 gather")
    d = _mx_problem([7, 0, 300, 9], 256, 512, seed=5, T=120, k=3)
    want = omoe.grouped_gemm(d["A"], d["offsets"], d["W"], "swiglu")
    out, amax = _run(d, ops.EPI_SWIGLU, torch.float32, want_amax=True)
    got = np_(out)
    assert rel_fro(got, want) < 1e-5
    assert np_(amax)[0] == np.abs(got).max()


def test_mxfp4_nan_weight_group():
    """A NaN in an MXFP4 weight row gives its 32-group the NaN scale 0xFF; the oracle's outputs
    of that weight row are NaN, and so must the scaled matrix cores' be."""
    say("mxfp4 nan weight")
    d = _mx_problem([100], 256, 256, seed=31)
    w = inputs.random_fp32((256, 256), 31, std=0.02)
    w[7, 40] = float("nan")
    wp, ws = ops.mxfp4_quantize(w.unsqueeze(0).to(DEV))
    assert np_(ws)[0, 7, 1] == 0xFF
    d["wt"] = ops.mxfp4_weights_tile(wp, ws)
    d["W"] = [omx.dequantize(np_(wp[0]), np_(ws[0]))]
    want = omoe.grouped_gemm(d["A"], d["offsets"], d["W"], "none")
    got = np_(_run(d, ops.EPI_NONE, torch.float32))
    assert np.isnan(want[:, 7]).all()
    assert np.array_equal(np.isnan(got), np.isnan(want))
    fin = np.isfinite(want)
    assert rel_fro(got[fin], want[fin]) < 1e-5


def test_grouped_gemm_mxfp4_rejects_unsupported_nw():
    d = _mx_problem([20], 256, 256, seed=3)
    wt = ops.MxTiledWeights(d["wt"].codes, d["wt"].scales, 160, 256)   # Nw = 160: not a multiple of 256
    t = lambda x: torch.from_numpy(x).to(DEV)
    with pytest.raises(_lib.NVFP4MoEError) as ei:
        ops.moe_grouped_gemm_mxfp4(ops.EPI_NONE, d["ap"], d["as_"], wt, t(d["offsets"]), t(d["active"]),
                                   t(d["n_active"]), rows=d["rows"])
    assert ei.value.status == _lib.ERR_UNSUPPORTED


# ------------------------------------------------------------------ the MXFP4 layer
def _mx_oracle_experts(w):
    return (lambda e: (np_(w.w13_packed[e]), np_(w.w13_scales[e])),
            lambda e: (np_(w.w2_packed[e]), np_(w.w2_scales[e])))


def test_tiny_mxfp4_layer_end_to_end():
    from nvfp4_block_scaled_moe_amd import layer
    wl = inputs.WORKLOADS["tiny"]
    say("tiny mxfp4 layer")
    w = layer.quantize_experts_mxfp4(wl, DEV)
    x = inputs.activations_bf16(wl)
    lg = inputs.router_logits(wl)
    out, st = layer.moe_forward_mxfp4(x.to(DEV), lg.to(DEV), wl.k, w, keep=True)
    torch.cuda.synchronize()
    w13, w2 = _mx_oracle_experts(w)
    for e in range(wl.E):   # weight quantization bit-exact
        po, so = omx.quantize(inputs.expert_weight_fp32(wl, "w13", e, DEV).cpu().numpy())
        assert np.array_equal(w13(e)[0], po) and np.array_equal(w13(e)[1], so)
    want, ost = omoe.moe_layer(x.float().numpy(), lg.numpy(), wl.k, w13, w2, mode="mxfp4", return_stages=True)
    got = np_(out)
    assert_finite(got)
    assert np.array_equal(np_(st["topk_ids"]), ost["ids"])
    assert np.array_equal(np_(st["xq"]), ost["xq"][0]) and np.array_equal(np_(st["xs"]), ost["xq"][1])
    r = rel_fro(got, want)
    say("tiny mxfp4 layer rel err", r)
    assert r <= W4A4_TOL


def test_prefill_mxfp4_layer_full_size():
    """The prefill workload (8192 tokens, 256 experts, top-8, H=7168, F=2048, Zipf routing)
    in MXFP4, exactly the calls the benchmark times: routing in full, activation and h codes
    in full (h's codes from the quantizing epilogue against the oracle's quantization of the
    fp32 h of the unquantized call), both GEMMs on every active expert (every 64-row block's
    edge rows x 4 columns of every 64-column block), the reduce in full, element by element."""
    from nvfp4_block_scaled_moe_amd import layer
    wl = inputs.WORKLOADS["prefill"]
    T = wl.T
    say("full-size mxfp4 layer", wl.name, T)
    w = layer.quantize_experts_mxfp4(wl, DEV)
    x = inputs.activations_bf16(wl, T).to(DEV)
    lg = inputs.router_logits(wl, T)
    out, st = layer.moe_forward_mxfp4(x, lg.to(DEV), wl.k, w, keep=True)
    # the float32 h of the same up/gate GEMM without the quantized epilogue
    st["h"] = ops.moe_grouped_gemm_mxfp4(ops.EPI_SWIGLU, st["xq"], st["xs"], w.w13_t,
                                         st["expert_offsets"], st["active_experts"], st["n_active"],
                                         gather_index=st["sorted_slot"], gather_div=wl.k, rows=T * wl.k,
                                         out_dtype=torch.float32)
    torch.cuda.synchronize()
    ids, rw = omoe.route(lg.numpy(), wl.k)
    perm = omoe.permute(ids, wl.E)
    assert np.array_equal(np_(st["topk_ids"]), ids)
    for key, ref in [("expert_offsets", perm["offsets"]), ("sorted_slot", perm["sorted_slot"]),
                     ("slot_to_row", perm["slot_to_row"])]:
        assert np.array_equal(np_(st[key]), ref), key
    xq = omx.quantize(np_(x).astype(np.float32))
    assert np.array_equal(np_(st["xq"]), xq[0]) and np.array_equal(np_(st["xs"]), xq[1])
    h32 = np_(st["h"]).astype(np.float32)
    hq = omx.quantize(h32)
    assert np.array_equal(np_(st["hq"]), hq[0]) and np.array_equal(np_(st["hs"]), hq[1])
    A_all = omx.dequantize(*xq)
    y = np_(st["y"])
    assert_finite(h32, y)
    offsets = perm["offsets"]
    tok = perm["sorted_slot"] // wl.k
    counts = np.diff(offsets)
    act = np.nonzero(counts)[0]
    order = act[np.argsort(counts[act], kind="stable")]
    for e in sorted({int(order[-1]), int(order[len(order) // 2]), int(order[0])}):   # weight codes
        po, so = omx.quantize(inputs.expert_weight_fp32(wl, "w13", e, DEV).cpu().numpy())
        assert np.array_equal(np_(w.w13_packed[e]), po) and np.array_equal(np_(w.w13_scales[e]), so)

    def deq(packed, scales):
        def f(e, idx):
            ix = torch.from_numpy(np.asarray(idx, dtype=np.int64)).to(DEV)
            return omx.dequantize(np_(packed[e][ix]), np_(scales[e][ix]))
        return f
    check_every_expert(offsets, tok, A_all, h32, y, lambda rows: omx.dequantize(hq[0][rows], hq[1][rows]),
                       deq(w.w13_packed, w.w13_scales), deq(w.w2_packed, w.w2_scales), wl.F, wl.H,
                       lambda v: v, tol_h=1e-5, seed=T)
    got = np_(out)
    assert_finite(got)
    assert_reduce_elementwise(got, y, perm["slot_to_row"], np_(st["topk_w"]))
