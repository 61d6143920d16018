"""Pins of the MoE-layer oracle against things other than itself (CPU only).

Router: iterative arg-max selection (a different algorithm from the oracle's
sort), torch.softmax, closed-form special cases. Permutation: numpy's stable
argsort and invariants. GEMM: exact rational arithmetic (fractions) on tiny
shapes. SwiGLU: closed forms and torch.nn.functional.silu. Layer: reduction
to a dense SwiGLU FFN computed by torch in float64. Roundings: torch's
float32 -> bfloat16 / float8_e4m3fn casts and exact rational rounding.
"""
from fractions import Fraction

import numpy as np
import pytest
import torch

from oracle import moe, mxfp4, nvfp4


# ------------------------------------------------------------------ rounding
def test_bf16_round_matches_torch_on_float32_inputs():
    rng = np.random.default_rng(10)
    x = np.concatenate([
        rng.standard_normal(20000) * np.exp2(rng.uniform(-140, 120, 20000)),
        (np.arange(1, 2000) * 2.0 ** -133),                 # subnormal bf16 range
        [3.3895313892515355e38, 3.39e38, -3.4e38],          # max and overflow
    ]).astype(np.float32)
    # exact ties: 8 significant bits plus a trailing 1
    ties = (np.arange(256, 512) * 2 + 1).astype(np.float32) * np.float32(2.0 ** -9)
    x = np.concatenate([x, ties, -ties])
    ref = torch.from_numpy(x).to(torch.bfloat16).double().numpy()
    ours = moe.bf16_round(x.astype(np.float64))
    assert np.array_equal(np.isinf(ref), np.isinf(ours))
    fin = np.isfinite(ref)
    assert np.array_equal(ref[fin], ours[fin])


def test_bf16_round_float64_inputs_against_exact_rationals():
    rng = np.random.default_rng(11)
    x = rng.standard_normal(400) * np.exp2(rng.uniform(-20, 20, 400))
    got = moe.bf16_round(x)
    for xi, gi in zip(x, got):
        fx = Fraction(float(xi))
        m, e = np.frexp(xi)
        q = Fraction(2) ** (int(e) - 8)                     # spacing of bf16 at xi
        lo = (fx / q).__floor__() * q
        hi = lo + q
        d_lo, d_hi = fx - lo, hi - fx
        if d_lo < d_hi:
            want = lo
        elif d_hi < d_lo:
            want = hi
        else:
            want = lo if (lo / q) % 2 == 0 else hi
        assert Fraction(float(gi)) == want


# -------------------------------------------------------------------- router
def _topk_by_iterated_argmax(row, k):
    r = row.astype(np.float64).copy()
    out = []
    for _ in range(k):
        i = int(np.argmax(r))           # first maximum = lowest id among ties
        out.append(i)
        r[i] = -np.inf
    return out


@pytest.mark.parametrize("T,E,k", [(16, 8, 2), (7, 256, 8), (3, 512, 22), (5, 8, 8), (4, 1, 1)])
def test_route_against_iterated_argmax_and_torch_softmax(T, E, k):
    rng = np.random.default_rng(T * 1000 + E + k)
    lg = rng.standard_normal((T, E)).astype(np.float32)
    lg[0, : min(E, 4)] = lg[0].max() + 1.0            # ties at the top of row 0
    lg[-1, -min(E, 3):] = 0.25                        # ties elsewhere
    ids, w = moe.route(lg, k)
    p = torch.softmax(torch.from_numpy(lg).double(), dim=1).numpy()
    for t in range(T):
        sel = _topk_by_iterated_argmax(lg[t], k)
        assert ids[t].tolist() == sel
        ref = p[t, sel] / p[t, sel].sum()
        np.testing.assert_allclose(w[t], ref, rtol=1e-13, atol=0)
    np.testing.assert_allclose(w.sum(1), 1.0, rtol=1e-13)


def test_route_special_cases():
    ids, w = moe.route(np.zeros((3, 16), np.float32), 4)
    assert ids.tolist() == [[0, 1, 2, 3]] * 3
    np.testing.assert_allclose(w, 0.25, rtol=0, atol=1e-15)
    lg = np.random.default_rng(0).standard_normal((2, 6)).astype(np.float32)
    ids, w = moe.route(lg, 6)                          # k = E keeps the full softmax
    full = torch.softmax(torch.from_numpy(lg).double(), 1).numpy()
    for t in range(2):
        assert sorted(ids[t].tolist()) == list(range(6))
        np.testing.assert_allclose(w[t], full[t, ids[t]], rtol=1e-13)
    ids, w = moe.route(lg, 1)
    assert np.all(w == 1.0) and ids[:, 0].tolist() == np.argmax(lg, 1).tolist()


# --------------------------------------------------------------- permutation
@pytest.mark.parametrize("T,E,k", [(16, 8, 2), (1, 256, 8), (64, 512, 22), (300, 4, 3)])
def test_permute_matches_stable_argsort(T, E, k):
    rng = np.random.default_rng(T + E + k)
    ids = np.stack([rng.choice(E, size=k, replace=False) for _ in range(T)]).astype(np.int32)
    p = moe.permute(ids, E)
    flat = ids.reshape(-1)
    order = np.argsort(flat, kind="stable")
    assert np.array_equal(p["sorted_slot"], order)
    counts = np.bincount(flat, minlength=E)
    assert np.array_equal(p["counts"], counts)
    assert np.array_equal(p["offsets"], np.concatenate([[0], np.cumsum(counts)]))
    assert p["offsets"][-1] == T * k
    assert np.array_equal(p["active"], np.unique(flat))
    assert np.array_equal(p["sorted_slot"][p["slot_to_row"]], np.arange(T * k))
    assert np.all(np.diff(flat[p["sorted_slot"]]) >= 0)


# --------------------------------------------------------------------- GEMMs
def _nvfp4_random(rng, R, C):
    w = (rng.standard_normal((R, C)) * 0.02).astype(np.float32)
    return nvfp4.quantize(w)


def test_grouped_gemm_exact_rationals_tiny():
    rng = np.random.default_rng(20)
    E, K, N = 3, 32, 6
    offsets = np.array([0, 2, 2, 5])                    # expert 1 empty
    A = moe.bf16_round(rng.standard_normal((5, K)))
    Wq = [_nvfp4_random(rng, N, K) for _ in range(E)]
    W = [nvfp4.dequantize(*q) for q in Wq]
    got = moe.grouped_gemm(A, offsets, W)
    for e in range(E):
        for r in range(offsets[e], offsets[e + 1]):
            for n in range(N):
                exact = sum(Fraction(float(A[r, kk])) * Fraction(float(W[e][n, kk])) for kk in range(K))
                assert abs(Fraction(float(got[r, n])) - exact) <= abs(exact) * Fraction(1, 2 ** 48) + Fraction(1, 2 ** 80)


def test_dequantized_weights_are_exact_dyadics():
    rng = np.random.default_rng(21)
    packed, scales, g = _nvfp4_random(rng, 4, 64)
    W = nvfp4.dequantize(packed, scales, g)
    q = nvfp4.unpack_fp4(packed)
    for r in range(4):
        for c in range(64):
            e2 = Fraction(nvfp4.E2M1_TABLE[q[r, c]])
            e4 = Fraction(nvfp4.E4M3_TABLE[scales[r, c // 16]])
            assert Fraction(float(W[r, c])) == e2 * e4 * Fraction(float(g))


def test_swiglu_closed_forms():
    x = np.linspace(-30, 30, 601)
    s = moe.silu(x)
    assert moe.silu(np.array([0.0]))[0] == 0.0
    np.testing.assert_allclose(moe.silu(-x), s - x, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(s[x > 25], x[x > 25], rtol=1e-10)
    np.testing.assert_allclose(s, torch.nn.functional.silu(torch.from_numpy(x)).numpy(), rtol=1e-14)
    G = np.concatenate([x[None, :], np.ones((1, 601))], 1)           # gate first, up second
    np.testing.assert_allclose(moe.swiglu(G)[0], s, rtol=0)


def test_unpermute_reduce_gather_and_one_hot():
    T, k, H = 5, 3, 7
    rng = np.random.default_rng(30)
    s2r = rng.permutation(T * k)
    Y = np.zeros((T * k, H))
    for s in range(T * k):
        Y[s2r[s], s % H] = 1.0                                        # one-hot rows
    w = rng.random((T, k))
    out = moe.unpermute_reduce(Y, s2r, w)
    want = np.zeros((T, H))
    for t in range(T):
        for j in range(k):
            want[t, (t * k + j) % H] += w[t, j]
    np.testing.assert_array_equal(out, want)
    Y1 = rng.standard_normal((T, H))
    s1 = rng.permutation(T)
    np.testing.assert_array_equal(moe.unpermute_reduce(Y1, s1, np.ones((T, 1))), Y1[s1])


def test_layer_with_one_expert_is_a_dense_swiglu_ffn():
    rng = np.random.default_rng(40)
    T, H, F = 6, 64, 32
    x = moe.bf16_round(rng.standard_normal((T, H))).astype(np.float32)
    w13 = _nvfp4_random(rng, 2 * F, H)
    w2 = _nvfp4_random(rng, H, F)
    out, st = moe.moe_layer(x, np.zeros((T, 1), np.float32), 1, lambda e: w13, lambda e: w2,
                            return_stages=True)
    X = torch.from_numpy(x.astype(np.float64))
    W13 = torch.from_numpy(nvfp4.dequantize(*w13))
    W2 = torch.from_numpy(nvfp4.dequantize(*w2))
    G = X @ W13.T
    h = torch.nn.functional.silu(G[:, :F]) * G[:, F:]
    h = h.float().to(torch.bfloat16).double()    # h in float64 -> bf16 via float32 (may differ by a tie)
    ref = (h @ W2.T).float().to(torch.bfloat16).double().numpy()
    assert np.array_equal(st["perm"]["sorted_slot"], np.arange(T))
    rel = np.linalg.norm(out - ref) / np.linalg.norm(ref)
    assert rel < 4e-3                             # two bf16 roundings may differ by one ulp
    np.testing.assert_allclose(st["h_exact"], (torch.nn.functional.silu(G[:, :F]) * G[:, F:]).numpy(),
                               rtol=1e-12, atol=1e-15)


def test_layer_w4a4_uses_quantized_activations():
    rng = np.random.default_rng(41)
    T, E, k, H, F = 8, 4, 2, 64, 32
    x = moe.bf16_round(rng.standard_normal((T, H))).astype(np.float32)
    lg = rng.standard_normal((T, E)).astype(np.float32)
    W13 = [_nvfp4_random(rng, 2 * F, H) for _ in range(E)]
    W2 = [_nvfp4_random(rng, H, F) for _ in range(E)]
    out, st = moe.moe_layer(x, lg, k, lambda e: W13[e], lambda e: W2[e], mode="w4a4", return_stages=True)
    out16 = moe.moe_layer(x, lg, k, lambda e: W13[e], lambda e: W2[e], mode="w4a16")
    rel = np.linalg.norm(out - out16) / np.linalg.norm(out16)
    assert 0.03 < rel < 0.3                       # activation quantization noise is present
    xq = nvfp4.dequantize(*st["xq"])
    assert np.linalg.norm(xq - x) / np.linalg.norm(x) < 0.12


def test_layer_w4a4_with_one_expert_is_a_dense_nvfp4_ffn():
    """NVFP4 W4A4 layer with E = 1, k = 1 against a dense SwiGLU FFN computed by torch in
    float64: the token rows are NVFP4-quantized as one tensor (one dynamic global scale), the
    FFN's h is NVFP4-quantized again as one tensor with its own dynamic global scale, and both
    GEMMs take the dequantized operands. Rows of very different magnitude make a per-row
    global scale give visibly different codes, and h's re-quantization moves the output by
    far more than the output's bf16 rounding."""
    rng = np.random.default_rng(43)
    T, H, F = 6, 64, 64
    mag = np.array([1.0, 8.0, 0.1, 3.0, 0.5, 20.0])[:, None]
    x = moe.bf16_round(rng.standard_normal((T, H)) * mag).astype(np.float32)
    w13 = _nvfp4_random(rng, 2 * F, H)
    w2 = _nvfp4_random(rng, H, F)
    out, st = moe.moe_layer(x, np.zeros((T, 1), np.float32), 1, lambda e: w13, lambda e: w2,
                            mode="w4a4", return_stages=True)
    xq = nvfp4.quantize(x)
    X = torch.from_numpy(nvfp4.dequantize(*xq))
    W13 = torch.from_numpy(nvfp4.dequantize(*w13))
    W2 = torch.from_numpy(nvfp4.dequantize(*w2))
    G = X @ W13.T
    h = torch.nn.functional.silu(G[:, :F]) * G[:, F:]
    hq = nvfp4.quantize(h.float().numpy())
    ref = (torch.from_numpy(nvfp4.dequantize(*hq)) @ W2.T).float().to(torch.bfloat16).double().numpy()
    rel = np.linalg.norm(out - ref) / np.linalg.norm(ref)
    assert rel < 4e-3                             # bf16 output rounding may differ by one ulp
    ref_norm = np.linalg.norm(ref, axis=1)
    assert ref_norm.min() > 0
    row_rel = np.linalg.norm(out - ref, axis=1) / ref_norm
    assert row_rel.max() < 4e-3                   # small rows judged on their own scale
    assert np.mean(out != ref) < 0.02
    assert np.array_equal(st["xq"][0], xq[0]) and np.array_equal(st["xq"][1], xq[1])
    assert st["xq"][2] == xq[2]
    assert np.array_equal(st["hq"][0], hq[0]) and np.array_equal(st["hq"][1], hq[1])
    assert st["hq"][2] == hq[2]
    np.testing.assert_allclose(st["h_exact"], h.numpy(), rtol=1e-12, atol=1e-15)


def _mxfp4_random(rng, R, C):
    return mxfp4.quantize((rng.standard_normal((R, C)) * 0.02).astype(np.float32))


def test_layer_mxfp4_with_one_expert_is_a_dense_mxfp4_ffn():
    """MXFP4 layer with E = 1, k = 1: x and h MXFP4-quantized, the products and SwiGLU
    computed by torch in float64 from the dequantized operands."""
    rng = np.random.default_rng(42)
    T, H, F = 6, 64, 64
    x = moe.bf16_round(rng.standard_normal((T, H))).astype(np.float32)
    w13 = _mxfp4_random(rng, 2 * F, H)
    w2 = _mxfp4_random(rng, H, F)
    out, st = moe.moe_layer(x, np.zeros((T, 1), np.float32), 1, lambda e: w13, lambda e: w2,
                            mode="mxfp4", return_stages=True)
    X = torch.from_numpy(mxfp4.dequantize(*mxfp4.quantize(x)))
    W13 = torch.from_numpy(mxfp4.dequantize(*w13))
    W2 = torch.from_numpy(mxfp4.dequantize(*w2))
    G = X @ W13.T
    h = torch.nn.functional.silu(G[:, :F]) * G[:, F:]
    hq = torch.from_numpy(mxfp4.dequantize(*mxfp4.quantize(h.float().numpy())))
    ref = (hq @ W2.T).float().to(torch.bfloat16).double().numpy()
    assert np.array_equal(st["xq"][0], mxfp4.quantize(x)[0])
    rel = np.linalg.norm(out - ref) / np.linalg.norm(ref)
    assert rel < 4e-3                             # bf16 output rounding may differ by one ulp
    np.testing.assert_allclose(st["h_exact"], h.numpy(), rtol=1e-12, atol=1e-15)
    # h is re-quantized: the down GEMM's input sits on the MXFP4 grid, not on bf16's
    assert np.linalg.norm(st["h"] - st["h_exact"]) / np.linalg.norm(st["h_exact"]) > 0.02


def test_fp8_roundtrip_matches_torch_cast_path():
    rng = np.random.default_rng(50)
    x = (rng.standard_normal((32, 128)) * 3).astype(np.float32)
    got = moe.fp8_roundtrip_bf16(x)
    xt = torch.from_numpy(x)
    s = (xt.abs().max() / 448.0).float()
    q = (xt / s).clamp(-448, 448).to(torch.float8_e4m3fn).float()
    ref = (q * s).to(torch.bfloat16).double().numpy()
    np.testing.assert_array_equal(got, ref)


def test_fp8_roundtrip_nonfinite_inputs():
    x = np.array([[1.0, -2.0, np.inf, np.nan, -np.inf, 0.5]], dtype=np.float32)
    got = moe.fp8_roundtrip_bf16(x)
    assert got[0, 1] == -2.0 and got[0, 2] == 2.0 and got[0, 4] == -2.0   # +-Inf saturate to +-448 * s_a
    assert np.isnan(got[0, 3]) and got[0, 0] == 1.0 and got[0, 5] == 0.5
