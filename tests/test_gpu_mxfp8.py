"""GPU parity of the block-scaled FP8 (MXFP8) dense/grouped GEMM against the MXFP8 oracle.

Quantizer codes and scales and the tiled code storage must match bit for bit; the W8A8
grouped GEMM on the scaled FP8 matrix cores must match the float64 oracle fed the same
dequantized operands within MX8_TOL relative Frobenius in float32 output: products of two
E4M3 values carry up to 8 significant bits, so the matrix core's float32 sums of each
32-element block are not exact (measured ~1.4e-5 at K = 640), unlike FP4 products, and
the bound allows for that rounding over K (no quantization error enters: both sides use
the same codes).
"""
import numpy as np
import pytest
import torch

from nvfp4_block_scaled_moe_amd import inputs, ops
from oracle import moe as omoe
from oracle import mxfp8 as om8
from tests.gpu_util import assert_finite, np_, rel_fro, say
from tests.test_gpu_mxfp4 import _mx_tile_reference, _special

pytestmark = pytest.mark.gpu
DEV = "cuda"
MX8_TOL = 1e-4


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    torch.cuda.init()


@pytest.mark.parametrize("R,C,dt", [(4, 128, torch.float32), (33, 96, torch.float32), (64, 2048, torch.float32),
                                    (5, 4096, torch.bfloat16), (2, 128, torch.bfloat16)])
def test_mxfp8_quantize_bit_exact(R, C, dt):
    say("mx8 quantize", R, C, dt)
    x = _special(R, C, R + C + 5)
    if C >= 128 and R > 1:
        x[1, 96:128] = 500.0                     # saturation at 448 * 2^e
        x[1, 97] = 272.0 / 256.0 * 500.0 / 2.0    # an element between grid points
    x = x.to(dt)
    c, s = ops.mxfp8_quantize(x.to(DEV))
    torch.cuda.synchronize()
    wc, ws = om8.quantize(x.float().numpy())
    assert np.array_equal(np_(c), wc)
    assert np.array_equal(np_(s), ws)


def _codes8_reference(codes):
    """Index-by-index transcription of the MXFP8 code tiles (include/nvfp4moe.h): lane
    16 g + r holds columns 16 g .. +15 and 64 + 16 g .. +15 of the chunk."""
    B, R, C = codes.shape
    nch = -(-C // 128)
    t = np.zeros((B, R // 16, nch, 64, 32), np.uint8)
    for b in range(B):
        for row in range(R):
            rb, r = divmod(row, 16)
            for c in range(nch):
                for g in range(4):
                    for h in range(2):
                        k0 = 128 * c + 16 * g + 64 * h
                        if k0 < C:
                            t[b, rb, c, 16 * g + r, 16 * h:16 * h + 16] = codes[b, row, k0:k0 + 16]
    return t.reshape(B, -1)


@pytest.mark.parametrize("B,R,C", [(1, 16, 32), (2, 48, 160), (1, 32, 2176)])
def test_mxfp8_weights_tile_bit_exact(B, R, C):
    say("mx8 tile", B, R, C)
    rng = np.random.default_rng(B * 5 + R + C)
    codes = rng.integers(0, 256, size=(B, R, C), dtype=np.uint8)
    scales = rng.integers(0, 256, size=(B, R, C // 32), dtype=np.uint8)
    t = ops.mxfp8_weights_tile(torch.from_numpy(codes).to(DEV), torch.from_numpy(scales).to(DEV))
    torch.cuda.synchronize()
    assert np.array_equal(np_(t.codes), _codes8_reference(codes))
    assert np.array_equal(np_(t.scales), _mx_tile_reference(np.zeros((B, R, C // 2), np.uint8), scales))


def _problem(counts, Nw, K, seed, T=None, k=None):
    E = len(counts)
    offsets = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    rows = int(offsets[-1])
    act = [e for e in range(E) if counts[e] > 0]
    active = np.array(act + [-1] * (E - len(act)), np.int32)
    w = torch.stack([inputs.random_fp32((Nw, K), seed + 17 * e, std=0.02) for e in range(E)])
    wc, ws = ops.mxfp8_quantize(w.to(DEV))
    nA = rows if T is None else T
    a = inputs.random_fp32((nA, K), seed + 1).to(torch.bfloat16)
    ac, as_ = ops.mxfp8_quantize(a.to(DEV))
    A = om8.dequantize(np_(ac), np_(as_))
    gidx = None
    if T is not None:
        gidx = np.random.default_rng(seed).integers(0, T * k, size=rows).astype(np.int32)
        A = A[gidx // k]
    return dict(rows=rows, offsets=offsets, active=active, n_active=np.array([len(act)], np.int32),
                wt=ops.mxfp8_weights_tile(wc, ws), ac=ac, as_=as_, A=A, gidx=gidx, gdiv=k or 1,
                W=[om8.dequantize(np_(wc[e]), np_(ws[e])) for e in range(E)])


def _run(d, epi, out_dtype=torch.float32, want_amax=False):
    t = lambda x: torch.from_numpy(x).to(DEV)
    res = ops.moe_grouped_gemm_mxfp8(epi, d["ac"], d["as_"], d["wt"], t(d["offsets"]), t(d["active"]),
                                     t(d["n_active"]), rows=d["rows"], out_dtype=out_dtype,
                                     gather_index=None if d["gidx"] is None else t(d["gidx"]),
                                     gather_div=d["gdiv"], want_amax=want_amax)
    torch.cuda.synchronize()
    return res


MX8_CASES = [
    # counts per expert, Nw, K (m-tiles of 64 rows)
    ([150, 0, 40, 70], 512, 640),        # ragged m-tiles, a 0-row expert, K % 128 != 0
    ([64], 256, 2048),                   # one full m-tile, one scale window
    ([300, 7], 256, 4096 + 96),          # two scale windows and a partial one
    ([1, 2, 3, 200], 768, 256),          # three row tiles, tiny experts
]


@pytest.mark.parametrize("ksplit", [None, "3"])
@pytest.mark.parametrize("counts,Nw,K", MX8_CASES)
def test_grouped_gemm_mxfp8(counts, Nw, K, ksplit, monkeypatch):
    say("gemm mxfp8", counts, Nw, K, ksplit)
    if ksplit:
        monkeypatch.setenv("NVFP4MOE_MX_KSPLIT", ksplit)
    d = _problem(counts, Nw, K, seed=Nw + K + 3)
    for epi in (ops.EPI_NONE, ops.EPI_SWIGLU):
        want = omoe.grouped_gemm(d["A"], d["offsets"], d["W"], "swiglu" if epi else "none")
        got = np_(_run(d, epi))
        assert_finite(got)
        r = rel_fro(got, want)
        say("rel err", r)
        assert r < MX8_TOL, r       # identical operands on both sides: only float32 summation differs


@pytest.mark.parametrize("group,ksplit", [("3", "1"), ("16", "1"), ("4", "3")])
def test_grouped_gemm_mxfp8_tile_groups(group, ksplit, monkeypatch):
    """Experts with several groups of 64-row m-tiles (the last group shorter, the last m-tile
    ragged), row-tile-major within a group, with and without K slices."""
    counts = [700, 0, 200, 65]           # 11, 0, 4 and 2 m-tiles of 64 rows
    say("gemm mxfp8 tile groups", group, ksplit)
    monkeypatch.setenv("NVFP4MOE_MX_GROUP", group)
    monkeypatch.setenv("NVFP4MOE_MX_KSPLIT", ksplit)
    d = _problem(counts, 512, 640, seed=93)
    for epi in (ops.EPI_NONE, ops.EPI_SWIGLU):
        want = omoe.grouped_gemm(d["A"], d["offsets"], d["W"], "swiglu" if epi else "none")
        got = np_(_run(d, epi))
        assert_finite(got)
        assert rel_fro(got, want) < MX8_TOL


def test_grouped_gemm_mxfp8_gather_and_amax():
    say("gemm mxfp8 gather")
    d = _problem([7, 0, 300, 9], 256, 512, seed=9, T=120, k=3)
    want = omoe.grouped_gemm(d["A"], d["offsets"], d["W"], "swiglu")
    out, amax = _run(d, ops.EPI_SWIGLU, want_amax=True)
    got = np_(out)
    assert rel_fro(got, want) < MX8_TOL
    assert np_(amax)[0] == np.abs(got).max()


def test_dense_mxfp8_gemm_full_size():
    """The dense GEMM M=512, N=2048, K=6144 in MXFP8 (K split on its own), full output."""
    wl = inputs.WORKLOADS["dense"]
    say("dense mxfp8")
    wc, ws = ops.mxfp8_quantize(inputs.expert_weight_fp32(wl, "dense", 0, DEV).unsqueeze(0))
    x = inputs.activations_bf16(wl).to(DEV)
    ac, as_ = ops.mxfp8_quantize(x)
    one = lambda v: torch.tensor(v, dtype=torch.int32, device=DEV)
    out = ops.moe_grouped_gemm_mxfp8(ops.EPI_NONE, ac, as_, ops.mxfp8_weights_tile(wc, ws), one([0, wl.T]),
                                     one([0]), one([1]), out_dtype=torch.float32)
    torch.cuda.synchronize()
    want = om8.dequantize(np_(ac), np_(as_)) @ om8.dequantize(np_(wc[0]), np_(ws[0])).T
    got = np_(out)
    assert_finite(got)
    r = rel_fro(got, want)
    say("dense mxfp8 rel err", r)
    assert r < MX8_TOL
