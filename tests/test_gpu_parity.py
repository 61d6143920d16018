"""GPU parity: every C ABI call against the oracle on the same seeded inputs.

Integer/byte outputs (codes, scales, ids, offsets, permutation) must match bit for bit;
floating-point outputs must be within the stated relative Frobenius bounds (W4A16 1e-3,
W4A4 2e-2) of the float64 oracle fed identical dequantized operands, with the oracle
rounded to the output dtype at the same points. Every GPU output is also scanned for
NaN/Inf.
"""
import numpy as np
import pytest
import torch

from nvfp4_block_scaled_moe_amd import inputs, ops
from oracle import moe as omoe
from oracle import nvfp4 as onv
from tests.gpu_util import assert_finite, assert_reduce_elementwise, np_, rel_fro, say

pytestmark = pytest.mark.gpu
DEV = "cuda"
W4A16_TOL = 1e-3
W4A4_TOL = 2e-2


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    torch.cuda.init()


# ------------------------------------------------------------------ quantize
def _special_matrix(R, C, seed):
    x = inputs.random_fp32((R, C), seed, std=0.02)
    x[0, :16] = 0.0
    x[0, 3] = -0.0
    if R > 1 and C >= 64:
        x[1, 16:32] *= 1e-7                       # subnormal E4M3 scales
        x[1, 40] = float("nan")
        x[1, 50] = float("inf")
        x[1, 33] = 5.0                            # sets the global scale
    return x


@pytest.mark.parametrize("R,C,dt", [(16, 64, torch.float32), (33, 96, torch.float32),
                                    (128, 6144, torch.float32), (7, 32, torch.bfloat16),
                                    (256, 2048, torch.bfloat16)])
def test_quantize_bit_exact(R, C, dt):
    say("quantize", R, C, dt)
    x = _special_matrix(R, C, R * 1000 + C).to(dt)
    p, s, g = ops.nvfp4_quantize(x.to(DEV))
    torch.cuda.synchronize()
    po, so, go = onv.quantize(x.float().numpy())
    assert np.array_equal(np_(s), so)
    assert np.array_equal(np_(p), po)
    assert np_(g)[0] == go


def test_quantize_batched_static_and_amax_paths():
    say("quantize batched / g_in / amax_in")
    x = torch.stack([inputs.random_fp32((24, 128), 100 + b, std=0.02 * (b + 1)) for b in range(3)])
    p, s, g = ops.nvfp4_quantize(x.to(DEV))
    gs = torch.tensor([1e-4, 3e-5, 2.0 ** -12], dtype=torch.float32)
    p2, s2, g2 = ops.nvfp4_quantize(x.to(DEV), g=gs.to(DEV))
    amax = x.abs().amax(dim=(1, 2))
    p3, s3, g3 = ops.nvfp4_quantize(x.to(DEV), amax=amax.to(DEV))
    torch.cuda.synchronize()
    for b in range(3):
        po, so, go = onv.quantize(x[b].numpy())
        assert np.array_equal(np_(p[b]), po) and np.array_equal(np_(s[b]), so) and np_(g)[b] == go
        assert np.array_equal(np_(p3[b]), po) and np.array_equal(np_(s3[b]), so) and np_(g3)[b] == go
        po2, so2, _ = onv.quantize(x[b].numpy(), g=gs[b].item())
        assert np.array_equal(np_(p2[b]), po2) and np.array_equal(np_(s2[b]), so2)
        assert np_(g2)[b] == np.float32(gs[b].item())


# ------------------------------------------------------------------ weight tiling
def _tile_reference(packed, scales):
    """The tiled storage written out index by index from its definition (numpy, no kernel
    code): codes tile (rb, c) lane 16g+r = codes of columns 128c+32g..+31 of row 16rb+r;
    scales tile (rb, w) lane 16g+r byte 2u(+1) = scales of columns 128(8w+u)+32g(+16)."""
    B, R, Ch = packed.shape
    C = 2 * Ch
    nch, nwin = -(-C // 128), -(-C // 1024)
    codes = np.zeros((B, R // 16, nch, 64, 16), np.uint8)
    sc = np.zeros((B, R // 16, nwin, 64, 16), np.uint8)
    for b in range(B):
        for row in range(R):
            rb, r = divmod(row, 16)
            for g in range(4):
                lane = 16 * g + r
                for c in range(nch):
                    k0 = 128 * c + 32 * g
                    if k0 < C:
                        codes[b, rb, c, lane] = packed[b, row, k0 // 2:k0 // 2 + 16]
                for w in range(nwin):
                    for u in range(8):
                        k0 = 128 * (8 * w + u) + 32 * g
                        if k0 < C:
                            sc[b, rb, w, lane, 2 * u:2 * u + 2] = scales[b, row, k0 // 16:k0 // 16 + 2]
    return codes.reshape(B, -1), sc.reshape(B, -1)


@pytest.mark.parametrize("B,R,C", [(1, 16, 32), (2, 48, 160), (3, 32, 1056), (1, 64, 2048)])
def test_weights_tile_bit_exact(B, R, C):
    say("tile", B, R, C)
    rng = np.random.default_rng(B * 7 + R + C)
    packed = rng.integers(0, 256, size=(B, R, C // 2), dtype=np.uint8)
    scales = rng.integers(0, 256, size=(B, R, C // 16), dtype=np.uint8)
    g = torch.arange(1, B + 1, dtype=torch.float32, device=DEV)
    t = ops.nvfp4_weights_tile(torch.from_numpy(packed).to(DEV), torch.from_numpy(scales).to(DEV), g)
    torch.cuda.synchronize()
    want_c, want_s = _tile_reference(packed, scales)
    assert np.array_equal(np_(t.codes), want_c)
    assert np.array_equal(np_(t.scales), want_s)
    assert (t.R, t.C, t.B) == (R, C, B) and np.array_equal(np_(t.g), np_(g))


@pytest.mark.parametrize("B,R,C,dt,gmode", [(1, 16, 32, torch.float32, "dyn"), (2, 48, 160, torch.bfloat16, "dyn"),
                                             (3, 32, 1056, torch.float32, "static"), (2, 64, 2048, torch.float32, "amax"),
                                             (4, 256, 6144, torch.bfloat16, "dyn")])
def test_quantize_tiled_layout_bit_exact(B, R, C, dt, gmode):
    """nvfp4_quantize with the tiled layout writes exactly the bytes of the row-major quantize
    followed by the index-by-index tiling transcription (padding zeros past C included), and
    the row-major codes are the oracle's; NaN/Inf/zero groups included."""
    say("quantize tiled", B, R, C, dt, gmode)
    x = torch.stack([_special_matrix(R, C, 500 + 13 * b + C) for b in range(B)]).to(dt)
    kw = {}
    if gmode == "static":
        kw["g"] = torch.tensor([0.01 * (b + 1) for b in range(B)], dtype=torch.float32, device=DEV)
    elif gmode == "amax":
        xf = x.float()
        kw["amax"] = torch.where(xf.isfinite(), xf.abs(), torch.zeros_like(xf)).amax(dim=(1, 2)).to(DEV)
    p, sc, g = ops.nvfp4_quantize(x.to(DEV), **kw)
    t = ops.nvfp4_quantize(x.to(DEV), tiled=True, **kw)
    torch.cuda.synchronize()
    want_c, want_s = _tile_reference(np_(p), np_(sc))
    assert np.array_equal(np_(t.codes), want_c)
    assert np.array_equal(np_(t.scales), want_s)
    assert torch.equal(t.g, g) and (t.R, t.C, t.B) == (R, C, B)
    for b in range(B):
        po, so, go = onv.quantize(x[b].float().numpy(), None if gmode != "static" else np_(kw["g"])[b])
        assert np.array_equal(np_(p[b]), po) and np.array_equal(np_(sc[b]), so) and np_(g)[b] == go


@pytest.mark.parametrize("R,C", [(64, 256), (1, 8), (64, 2048), (1024, 512)])   # one-launch path, and the 3-launch one
def test_fp8_roundtrip_bit_exact(R, C):
    say("fp8 roundtrip", R, C)
    x = (inputs.random_fp32((R, C), 7) * 3).to(torch.bfloat16)
    x[0, 0] = float("inf")
    x[0, 1] = float("nan")
    x[0, 2] = -float("inf")
    x[R - 1, C - 1] = 1000.0 * (R * C > 1 << 14)          # the amax sits in the last vector (another slice)
    got = np_(ops.act_fp8_e4m3_roundtrip(x.to(DEV)))
    want = omoe.fp8_roundtrip_bf16(x.float().numpy())
    assert np.array_equal(np.isnan(got), np.isnan(want))
    m = ~np.isnan(want)
    assert np.array_equal(got[m], want[m])


# ------------------------------------------------------------------ routing
ROUTE_CASES = [(16, 8, 2, 0.0), (1, 256, 8, 0.0), (8, 256, 8, 0.0), (16, 256, 8, 0.0),
               (64, 256, 8, 0.0), (512, 256, 8, 0.0), (1, 512, 22, 0.0), (4, 512, 22, 0.0),
               (64, 512, 22, 0.0), (8192, 256, 8, 1.1), (5, 8, 8, 0.0), (3, 1, 1, 0.0),
               (37, 1024, 64, 0.0)]


@pytest.mark.parametrize("T,E,k,zipf", ROUTE_CASES)
def test_route_permute_bit_exact(T, E, k, zipf):
    say("route", T, E, k, zipf)
    wl = inputs.Workload("route_test", T=T, E=E, k=k, H=64, F=64, mode="w4a16", zipf=zipf)
    lg = inputs.router_logits(wl)
    if T >= 2:
        lg[1, :] = 0.25                           # an all-tie row
    _check_route(lg, k, E)


def _check_route(lg, k, E):
    r = ops.moe_route_permute(lg.to(DEV), k)
    torch.cuda.synchronize()
    ids, w = omoe.route(lg.numpy(), k)
    perm = omoe.permute(ids, E)
    assert np.array_equal(np_(r["topk_ids"]), ids)
    np.testing.assert_allclose(np_(r["topk_w"]), w, rtol=1e-6, atol=0)
    assert np.array_equal(np_(r["expert_offsets"]), perm["offsets"])
    assert np.array_equal(np_(r["sorted_slot"]), perm["sorted_slot"])
    assert np.array_equal(np_(r["slot_to_row"]), perm["slot_to_row"])
    na = int(np_(r["n_active"])[0])
    assert na == len(perm["active"])
    act = np_(r["active_experts"])
    assert np.array_equal(act[:na], perm["active"]) and np.all(act[na:] == -1)


@pytest.mark.parametrize("path", ["single", "multi"])
@pytest.mark.parametrize("T,E,k,zipf", [(8192, 256, 8, 1.1), (3000, 512, 22, 0.0), (37, 1024, 64, 0.0),
                                        (16, 8, 2, 0.0), (1, 256, 8, 0.0), (20000, 64, 7, 0.5)])
def test_both_permutations_bit_exact(path, T, E, k, zipf, monkeypatch):
    """The one-workgroup permutation and the two-launch one (chunks of 2048+ slots; 20000 x 7
    slots grow the chunks to keep at most 64), each forced, against the oracle."""
    say("permute", path, T, E, k, zipf)
    monkeypatch.setenv("NVFP4MOE_PERMUTE", path)
    wl = inputs.Workload("route_test", T=T, E=E, k=k, H=64, F=64, mode="w4a16", zipf=zipf)
    lg = inputs.router_logits(wl)
    if T >= 2:
        lg[1, :] = 0.25                           # an all-tie row
    _check_route(lg, k, E)


@pytest.mark.parametrize("router", ["sort", "wave"])
@pytest.mark.parametrize("T,E,k", [(5, 64, 64), (3, 100, 7), (300, 512, 22), (2, 1024, 64)])
def test_both_routers_bit_exact(router, T, E, k, monkeypatch):
    """Both router kernels (workgroup sort for few tokens, wave select for many) against
    the oracle, each forced on shapes the size rule would give to the other; ties planted."""
    say("router", router, T, E, k)
    monkeypatch.setenv("NVFP4MOE_ROUTER", router)
    lg = inputs.random_fp32((T, E), T * 31 + E)
    lg[0, : min(E, 8)] = 1.5                    # equal logits at the top of row 0
    if E > 40:
        lg[-1, 40] = -0.0
        lg[-1, 3] = 0.0
    r = ops.moe_route_permute(lg.to(DEV), k)
    torch.cuda.synchronize()
    ids, w = omoe.route(lg.numpy(), k)
    assert np.array_equal(np_(r["topk_ids"]), ids)
    np.testing.assert_allclose(np_(r["topk_w"]), w, rtol=1e-6, atol=0)


@pytest.mark.parametrize("select", ["rounds", "thresh"])
@pytest.mark.parametrize("T,E,k", [(16, 1024, 64), (16, 512, 22), (2, 64, 64), (7, 100, 7), (1, 256, 8),
                                   (1, 1, 1), (16, 8, 2), (3, 1000, 17), (1, 1024, 64), (1, 512, 22)])
def test_small_route_permute_bit_exact(T, E, k, select, monkeypatch):
    """Few tokens: routing and permutation in one workgroup and one launch, against the oracle,
    with each of the two top-k selections (k rounds of wave argmax; the threshold select);
    up to 64 slots the barrier-free permutation, above it the general one; ties, -0/+0 and an
    all-equal row planted."""
    say("small route", T, E, k, select)
    monkeypatch.setenv("NVFP4MOE_ROUTER", "small")
    monkeypatch.setenv("NVFP4MOE_SMALL_SELECT", select)
    lg = inputs.random_fp32((T, E), 7 * T + E + k)
    lg[0, : min(E, 9)] = 1.5                      # equal logits at the top of row 0
    if E > 40:
        lg[-1, 40] = -0.0
        lg[-1, 3] = 0.0
    if T >= 3:
        lg[1, :] = 0.25                           # an all-tie row
    _check_route(lg, k, E)


@pytest.mark.parametrize("T,E,k", [(1, 256, 8), (2, 1024, 32), (7, 100, 9), (3, 1000, 17)])
def test_small_permutation_paths_agree(T, E, k, monkeypatch):
    """Up to 64 slots: the barrier-free permutation and the general one give the same bits
    (both against the oracle)."""
    say("small permutation paths", T, E, k)
    monkeypatch.setenv("NVFP4MOE_ROUTER", "small")
    lg = inputs.random_fp32((T, E), 3 * T + E + k)
    lg[0, : min(E, 5)] = 0.5
    for full in ("full", "few"):
        monkeypatch.setenv("NVFP4MOE_SMALL_PERMUTE", full)
        _check_route(lg, k, E)


def test_route_permute_at_the_slot_limit():
    """T * k = 2^24 slots, the largest the ABI takes (262144 tokens, top-64 of 64 experts:
    k = E, every expert in every token): ids, offsets and the permutation bit-exact."""
    T, E, k = 1 << 18, 64, 64
    say("route at the slot limit", T, E, k)
    lg = inputs.random_fp32((T, E), 77)
    r = ops.moe_route_permute(lg.to(DEV), k)
    torch.cuda.synchronize()
    ids, w = omoe.route(lg.numpy(), k)
    assert np.array_equal(np_(r["topk_ids"]), ids)
    np.testing.assert_allclose(np_(r["topk_w"]), w, rtol=1e-6, atol=0)
    perm = omoe.permute(ids, E)
    assert np.array_equal(np_(r["expert_offsets"]), perm["offsets"])
    assert np.array_equal(np_(r["sorted_slot"]), perm["sorted_slot"])
    assert np.array_equal(np_(r["slot_to_row"]), perm["slot_to_row"])
    assert int(np_(r["n_active"])[0]) == E


def test_route_permute_is_deterministic():
    say("route determinism")
    wl = inputs.WORKLOADS["prefill"]
    lg = inputs.router_logits(wl).to(DEV)
    a = ops.moe_route_permute(lg, wl.k)
    b = ops.moe_route_permute(lg, wl.k)
    for key in a:
        assert torch.equal(a[key], b[key]), key


# ------------------------------------------------------------------ grouped GEMM
def _problem(counts, Nw, K, seed, mode=ops.W4A16, T=None, k=None):
    """Random grouped-GEMM problem with the given rows per expert (0 allowed)."""
    E = len(counts)
    offsets = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    rows = int(offsets[-1])
    active = np.array([e for e in range(E) if counts[e] > 0] + [-1] * (E - sum(c > 0 for c in counts)), np.int32)
    n_active = np.array([sum(c > 0 for c in counts)], np.int32)
    w = torch.stack([inputs.random_fp32((Nw, K), seed + 17 * e, std=0.02) for e in range(E)])
    wp, ws, wg = ops.nvfp4_quantize(w.to(DEV))
    d = dict(E=E, rows=rows, offsets=offsets, active=active, n_active=n_active, wp=wp, ws=ws, wg=wg,
             wt=ops.nvfp4_weights_tile(wp, ws, wg),
             W=[onv.dequantize(np_(wp[e]), np_(ws[e]), np_(wg)[e]) for e in range(E)])
    if T is None:
        a = inputs.random_fp32((rows, K), seed + 1).to(torch.bfloat16)
        d.update(a=a, gidx=None, gdiv=1, A=a.float().numpy().astype(np.float64))
    else:
        a = inputs.random_fp32((T, K), seed + 1).to(torch.bfloat16)
        gidx = np.random.default_rng(seed).integers(0, T * k, size=rows).astype(np.int32)
        d.update(a=a, gidx=torch.from_numpy(gidx), gdiv=k,
                 A=a.float().numpy().astype(np.float64)[gidx // k])
    if mode == ops.W4A4:
        aq, as_, ag = ops.nvfp4_quantize(a.to(DEV))
        d.update(aq=aq, as_=as_, ag=ag)
        Aq = onv.dequantize(np_(aq), np_(as_), np_(ag)[0])
        d["A"] = Aq if d["gidx"] is None else Aq[d["gidx"].numpy() // k]
    return d


def _run_gemm(d, mode, epi, out_dtype):
    t = lambda a: torch.from_numpy(a).to(DEV)
    kw = dict(rows=d["rows"], out_dtype=out_dtype, gather_div=d["gdiv"],
              gather_index=None if d["gidx"] is None else d["gidx"].to(DEV))
    if mode == ops.W4A4:
        a = d["aq"]
        kw.update(a_scales=d["as_"], a_g=d["ag"])
    else:
        a = d["a"].to(DEV)
    out = ops.moe_grouped_gemm_nvfp4(mode, epi, a, d["wt"], t(d["offsets"]), t(d["active"]),
                                     t(d["n_active"]), **kw)
    torch.cuda.synchronize()
    return np_(out)


@pytest.mark.parametrize("path", ["stream", "mfma"])
def test_gemm_nan_weight_group_stays_visible(path, monkeypatch):
    """A NaN in a weight row makes its 16-group's scale NaN (0x7F); every output of that
    weight row must be NaN, as in the oracle (NaN times a zero code), on both paths; the
    other outputs stay finite and match."""
    say("gemm nan weight", path)
    monkeypatch.setenv("NVFP4MOE_FORCE_PATH", path)
    counts, Nw, K = [200, 70], 256, 512
    E = len(counts)
    offsets = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    w = torch.stack([inputs.random_fp32((Nw, K), 91 + e, std=0.02) for e in range(E)])
    w[1, 5, 37] = float("nan")                   # expert 1, weight row 5
    wp, ws, wg = ops.nvfp4_quantize(w.to(DEV))
    a = inputs.random_fp32((int(offsets[-1]), K), 92).to(torch.bfloat16)
    t = lambda x: torch.from_numpy(x).to(DEV)
    out = np_(ops.moe_grouped_gemm_nvfp4(ops.W4A16, ops.EPI_NONE, a.to(DEV), ops.nvfp4_weights_tile(wp, ws, wg),
                                         t(offsets), t(np.arange(E, dtype=np.int32)), t(np.array([E], np.int32)),
                                         out_dtype=torch.float32))
    torch.cuda.synchronize()
    Wd = [onv.dequantize(np_(wp[e]), np_(ws[e]), np_(wg)[e]) for e in range(E)]
    want = omoe.grouped_gemm(a.float().numpy().astype(np.float64), offsets, Wd)
    assert np.isnan(want[offsets[1]:, 5]).all() and np.isfinite(np.delete(want, 5, axis=1)).all()
    assert np.array_equal(np.isnan(out), np.isnan(want))
    fin = np.isfinite(want)
    assert rel_fro(out[fin], want[fin]) < 1e-5


GEMM_CASES = [
    # counts per expert, Nw, K
    ([3, 0, 16, 17, 1], 64, 64),
    ([40, 0, 2], 160, 96),          # > 32 rows (two token passes), K % 128 != 0, Nw/16 = 10
    ([5, 33, 0, 0, 64], 1024, 256),
    ([1] * 8, 256, 512),
    ([12, 20], 96, 6144),
    ([1, 2, 3], 2048, 6144),
    ([2, 1], 64, 32768),            # longest row the bf16 prep holds in registers
    ([3, 5], 64, 32800),            # longer rows: the two-pass prep, K % 128 != 0
    ([600, 0, 500], 256, 2048),     # >= 1024 rows of <= 2048 columns: a wave per row in the prep
    ([700, 400], 128, 4096),        # ... <= 4096 columns
    ([1030], 64, 992),              # ... K % 128 != 0, rows % 4 != 0
]


@pytest.mark.parametrize("counts,Nw,K", GEMM_CASES)
@pytest.mark.parametrize("epi", [ops.EPI_NONE, ops.EPI_SWIGLU])
def test_grouped_gemm_w4a16(counts, Nw, K, epi):
    say("gemm w4a16", counts, Nw, K, epi)
    d = _problem(counts, Nw, K, seed=Nw + K)
    want = omoe.grouped_gemm(d["A"], d["offsets"], d["W"], "swiglu" if epi else "none")
    got32 = _run_gemm(d, ops.W4A16, epi, torch.float32)
    assert ops.last_dispatch() in (1, 2)
    assert_finite(got32)
    r = rel_fro(got32, want)
    assert r <= W4A16_TOL and r < 1e-5, r
    got16 = _run_gemm(d, ops.W4A16, epi, torch.bfloat16)
    assert_finite(got16)
    assert rel_fro(got16, omoe.bf16_round(want)) <= W4A16_TOL


@pytest.mark.parametrize("path", ["stream", "mfma"])
def test_grouped_gemm_max_experts(path, monkeypatch):
    """E = 1024 (the API maximum), most experts empty, a few with 1..300 rows; the active list
    and the device m-tile schedule then span the whole expert range."""
    say("gemm 1024 experts", path)
    monkeypatch.setenv("NVFP4MOE_FORCE_PATH", path)
    rng = np.random.default_rng(1024)
    counts = [0] * 1024
    for e, c in zip(rng.choice(1024, size=40, replace=False), rng.integers(1, 300, size=40)):
        counts[int(e)] = int(c)
    counts[1023] = 5
    d = _problem(counts, 256, 64, seed=77)
    want = omoe.grouped_gemm(d["A"], d["offsets"], d["W"], "swiglu")
    got = _run_gemm(d, ops.W4A16, ops.EPI_SWIGLU, torch.float32)
    assert ops.last_dispatch() == (ops.PATH_MFMA if path == "mfma" else ops.PATH_STREAM)
    assert rel_fro(got, want) < 1e-5


def test_grouped_gemm_w4a16_gather():
    say("gemm gather")
    d = _problem([7, 0, 30, 9], 128, 256, seed=5, T=20, k=3)
    want = omoe.grouped_gemm(d["A"], d["offsets"], d["W"], "swiglu")
    got = _run_gemm(d, ops.W4A16, ops.EPI_SWIGLU, torch.float32)
    assert rel_fro(got, want) < 1e-5


@pytest.mark.parametrize("counts,Nw,K", GEMM_CASES[:4])
def test_grouped_gemm_w4a4(counts, Nw, K):
    say("gemm w4a4", counts, Nw, K)
    d = _problem(counts, Nw, K, seed=3 * Nw + K, mode=ops.W4A4)
    for epi in (ops.EPI_NONE, ops.EPI_SWIGLU):
        want = omoe.grouped_gemm(d["A"], d["offsets"], d["W"], "swiglu" if epi else "none")
        got = _run_gemm(d, ops.W4A4, epi, torch.float32)
        assert_finite(got)
        r = rel_fro(got, want)
        assert r <= W4A4_TOL and r < 1e-5, r      # identical NVFP4 operands: exact products


def test_grouped_gemm_amax_output():
    say("gemm amax")
    d = _problem([9, 4], 64, 128, seed=11)
    t = lambda a: torch.from_numpy(a).to(DEV)
    out, amax = ops.moe_grouped_gemm_nvfp4(ops.W4A16, ops.EPI_SWIGLU, d["a"].to(DEV), d["wt"],
                                           t(d["offsets"]), t(d["active"]), t(d["n_active"]),
                                           out_dtype=torch.float32, want_amax=True)
    torch.cuda.synchronize()
    assert np_(amax)[0] == np.abs(np_(out)).max()


@pytest.mark.parametrize("counts", [[70, 0, 150], [700, 0, 500]])
@pytest.mark.parametrize("path,ksplit", [("stream", "1"), ("stream", "2"), ("mfma", "1"), ("mfma", "2")])
@pytest.mark.parametrize("out_dtype", [torch.float32, torch.bfloat16])
def test_grouped_gemm_amax_skips_nonfinite(path, ksplit, out_dtype, counts, monkeypatch):
    """out_amax is the max |out| over the finite values written: a NaN activation row and a
    row whose one nonzero element is Inf give NaN and +-Inf outputs, which must not reach the
    amax (the global scale of the quantized h depends on it); with a bf16 output, the amax of
    the rounded values. Both paths, with and without split K."""
    say("gemm amax non-finite", path, ksplit, out_dtype, counts)
    monkeypatch.setenv("NVFP4MOE_FORCE_PATH", path)
    monkeypatch.setenv("NVFP4MOE_STREAM_KSPLIT" if path == "stream" else "NVFP4MOE_LARGE_KSPLIT", ksplit)
    d = _problem(counts, 256, 2048, seed=13)
    a = d["a"].clone()
    a[3] = float("nan")
    a[100] = 0.0
    a[100, 17] = float("inf")
    t = lambda v: torch.from_numpy(v).to(DEV)
    out, amax = ops.moe_grouped_gemm_nvfp4(ops.W4A16, ops.EPI_NONE, a.to(DEV), d["wt"], t(d["offsets"]),
                                           t(d["active"]), t(d["n_active"]), rows=d["rows"], out_dtype=out_dtype,
                                           want_amax=True)
    torch.cuda.synchronize()
    o = np_(out).astype(np.float64)
    assert np.isnan(o[3]).all() and np.isinf(o[100]).any()
    fin = np.isfinite(o)
    assert np_(amax)[0] == np.abs(o[fin]).max()
    want = omoe.grouped_gemm(a.float().numpy().astype(np.float64), d["offsets"], d["W"])
    assert np.array_equal(np.isnan(o), np.isnan(want)) and np.array_equal(np.isinf(o), np.isinf(want))
    assert rel_fro(o[fin], want[fin]) < (1e-5 if out_dtype == torch.float32 else 4e-3)


# ------------------------------------------------------------------ grouped GEMM, large-M path
# The m-tiled MFMA path (128-row m-tiles from a device-side schedule) is chosen by size;
# these cases force it, so they also cover shapes the size rule would send elsewhere.
MFMA_CASES = [
    ([3, 0, 16, 17, 1], 256, 64),        # every m-tile ragged, K < one chunk
    ([200, 0, 130, 1], 512, 96),         # several m-tiles per expert, K % 128 != 0
    ([129, 127, 0, 300], 256, 1024),     # m-tile boundaries at 128 +- 1
    ([600], 768, 256),                   # one expert, three 256-row tiles (SwiGLU F = 384)
    ([1, 70, 3], 2048, 6144),            # full model K
]


@pytest.mark.parametrize("waves", ["8", "4"])
@pytest.mark.parametrize("counts,Nw,K", MFMA_CASES)
@pytest.mark.parametrize("mode", [ops.W4A16, ops.W4A4])
def test_grouped_gemm_mfma_path(counts, Nw, K, mode, waves, monkeypatch):
    say("gemm mfma", counts, Nw, K, mode, waves)
    monkeypatch.setenv("NVFP4MOE_FORCE_PATH", "mfma")
    monkeypatch.setenv("NVFP4MOE_LARGE_WAVES", waves)
    d = _problem(counts, Nw, K, seed=7 * Nw + K + mode, mode=mode)
    for epi in (ops.EPI_NONE, ops.EPI_SWIGLU):
        want = omoe.grouped_gemm(d["A"], d["offsets"], d["W"], "swiglu" if epi else "none")
        got32 = _run_gemm(d, mode, epi, torch.float32)
        assert ops.last_dispatch() == ops.PATH_MFMA
        assert_finite(got32)
        r = rel_fro(got32, want)
        assert r < 1e-5, r        # identical operands on both sides: only summation order differs
        got16 = _run_gemm(d, mode, epi, torch.bfloat16)
        assert rel_fro(got16, omoe.bf16_round(want)) <= W4A16_TOL


@pytest.mark.parametrize("waves", ["8", "4"])
def test_grouped_gemm_mfma_tile_shapes(waves, monkeypatch):
    """Both workgroup shapes of the MFMA path: 8 waves (256 weight rows) and 4 (128 rows,
    chosen for small grids)."""
    say("gemm mfma waves", waves)
    monkeypatch.setenv("NVFP4MOE_FORCE_PATH", "mfma")
    monkeypatch.setenv("NVFP4MOE_LARGE_WAVES", waves)
    d = _problem([150, 0, 40, 270], 512, 640, seed=31)
    for epi in (ops.EPI_NONE, ops.EPI_SWIGLU):
        want = omoe.grouped_gemm(d["A"], d["offsets"], d["W"], "swiglu" if epi else "none")
        got = _run_gemm(d, ops.W4A16, epi, torch.float32)
        assert ops.last_dispatch() == ops.PATH_MFMA
        assert rel_fro(got, want) < 1e-5


@pytest.mark.parametrize("ksplit", ["2", "4"])
@pytest.mark.parametrize("mode", [ops.W4A16, ops.W4A4])
def test_grouped_gemm_stream_split_k(ksplit, mode, monkeypatch):
    """The small-M kernel with K split into window-aligned slices (the decode regime at a
    handful of tokens): ragged last window, 0-row experts, > 32 rows (two passes), gather."""
    say("gemm stream split-k", ksplit, mode)
    monkeypatch.setenv("NVFP4MOE_FORCE_PATH", "stream")
    monkeypatch.setenv("NVFP4MOE_STREAM_KSPLIT", ksplit)
    d = _problem([3, 0, 40, 1, 9], 256, 3168, seed=int(ksplit) + 100 * mode, mode=mode, T=30, k=2)
    t = lambda a: torch.from_numpy(a).to(DEV)
    for epi in (ops.EPI_NONE, ops.EPI_SWIGLU):
        want = omoe.grouped_gemm(d["A"], d["offsets"], d["W"], "swiglu" if epi else "none")
        got = _run_gemm(d, mode, epi, torch.float32)
        assert ops.last_dispatch() == ops.PATH_STREAM
        assert_finite(got)
        assert rel_fro(got, want) < 1e-5
    kw = dict(rows=d["rows"], gather_index=d["gidx"].to(DEV), gather_div=d["gdiv"], out_dtype=torch.float32,
              want_amax=True)
    a = d["a"].to(DEV)
    if mode == ops.W4A4:
        a = d["aq"]
        kw.update(a_scales=d["as_"], a_g=d["ag"])
    out, amax = ops.moe_grouped_gemm_nvfp4(mode, ops.EPI_SWIGLU, a, d["wt"], t(d["offsets"]), t(d["active"]),
                                           t(d["n_active"]), **kw)
    torch.cuda.synchronize()
    assert np_(amax)[0] == np.abs(np_(out)).max()


@pytest.mark.parametrize("waves", ["8", "4"])
@pytest.mark.parametrize("ksplit", ["1", "2", "3"])
@pytest.mark.parametrize("mode", [ops.W4A16, ops.W4A4])
def test_grouped_gemm_mfma_split_k(ksplit, mode, waves, monkeypatch):
    """K split into slices of whole 1024-column windows (partial sums reduced in a fixed
    order by a second kernel that applies the epilogue); K = 3072 + 96 leaves a ragged last
    window; both workgroup shapes. amax of the output must equal max |out| exactly."""
    say("gemm mfma split-k", ksplit, mode, waves)
    monkeypatch.setenv("NVFP4MOE_FORCE_PATH", "mfma")
    monkeypatch.setenv("NVFP4MOE_LARGE_KSPLIT", ksplit)
    monkeypatch.setenv("NVFP4MOE_LARGE_WAVES", waves)
    d = _problem([300, 5, 0, 77], 512, 3168, seed=int(ksplit) + 10 * mode, mode=mode, T=250, k=2)
    t = lambda a: torch.from_numpy(a).to(DEV)
    for epi in (ops.EPI_NONE, ops.EPI_SWIGLU):
        want = omoe.grouped_gemm(d["A"], d["offsets"], d["W"], "swiglu" if epi else "none")
        got = _run_gemm(d, mode, epi, torch.float32)
        assert ops.last_dispatch() == ops.PATH_MFMA
        assert_finite(got)
        assert rel_fro(got, want) < 1e-5
    kw = dict(rows=d["rows"], gather_index=d["gidx"].to(DEV), gather_div=d["gdiv"], out_dtype=torch.bfloat16,
              want_amax=True)
    a = d["a"].to(DEV)
    if mode == ops.W4A4:
        a = d["aq"]
        kw.update(a_scales=d["as_"], a_g=d["ag"])
    out, amax = ops.moe_grouped_gemm_nvfp4(mode, ops.EPI_SWIGLU, a, d["wt"], t(d["offsets"]), t(d["active"]),
                                           t(d["n_active"]), **kw)
    torch.cuda.synchronize()
    o = np_(out).astype(np.float32)
    assert np_(amax)[0] == np.abs(o).max()        # the amax of the values as written (bf16)


@pytest.mark.parametrize("mode", [ops.W4A16, ops.W4A4])
def test_grouped_gemm_mfma_gather(mode, monkeypatch):
    say("gemm mfma gather", mode)
    monkeypatch.setenv("NVFP4MOE_FORCE_PATH", "mfma")
    d = _problem([7, 0, 300, 9], 256, 256, seed=5, T=120, k=3, mode=mode)
    want = omoe.grouped_gemm(d["A"], d["offsets"], d["W"], "swiglu")
    got = _run_gemm(d, mode, ops.EPI_SWIGLU, torch.float32)
    assert ops.last_dispatch() == ops.PATH_MFMA
    assert rel_fro(got, want) < 1e-5


@pytest.mark.parametrize("waves", ["8", "4"])
@pytest.mark.parametrize("ksplit", ["1", "2"])
@pytest.mark.parametrize("counts,K,T,k", [([300, 5, 0, 77], 3168, 250, 2), ([7, 0, 129, 9], 256, None, None)])
def test_grouped_gemm_mfma_w4a4_fp4_staging(waves, ksplit, counts, K, T, k, monkeypatch):
    """W4A4 on the large-M path with the NVFP4 activation rows decoded in the GEMM's staging
    (NVFP4MOE_LARGE_A4=1) instead of an f16 copy: the decoded values are the same exact
    products in the same accumulation order, so the output is bit-identical to the default
    path, and within 1e-5 of the oracle; gather, ragged and empty experts, K % 128 != 0."""
    say("gemm mfma w4a4 fp4 staging", waves, ksplit, counts, K)
    monkeypatch.setenv("NVFP4MOE_FORCE_PATH", "mfma")
    monkeypatch.setenv("NVFP4MOE_LARGE_WAVES", waves)
    monkeypatch.setenv("NVFP4MOE_LARGE_KSPLIT", ksplit)
    d = _problem(counts, 512, K, seed=77 + int(ksplit), mode=ops.W4A4, T=T, k=k)
    for epi in (ops.EPI_NONE, ops.EPI_SWIGLU):
        monkeypatch.delenv("NVFP4MOE_LARGE_A4", raising=False)
        ref = _run_gemm(d, ops.W4A4, epi, torch.float32)
        monkeypatch.setenv("NVFP4MOE_LARGE_A4", "1")
        got = _run_gemm(d, ops.W4A4, epi, torch.float32)
        assert ops.last_dispatch() == ops.PATH_MFMA
        assert np.array_equal(got, ref)
        want = omoe.grouped_gemm(d["A"], d["offsets"], d["W"], "swiglu" if epi else "none")
        assert rel_fro(got, want) < 1e-5


def test_grouped_gemm_path_choice_by_size(monkeypatch):
    """Mean rows per expert >= 64 selects the MFMA path; both paths agree on it."""
    say("gemm path choice")
    monkeypatch.delenv("NVFP4MOE_FORCE_PATH", raising=False)
    big = _problem([100, 60, 0, 96], 256, 256, seed=9)          # 256 rows over 4 experts
    got_auto = _run_gemm(big, ops.W4A16, ops.EPI_SWIGLU, torch.float32)
    assert ops.last_dispatch() == ops.PATH_MFMA
    monkeypatch.setenv("NVFP4MOE_FORCE_PATH", "stream")
    got_stream = _run_gemm(big, ops.W4A16, ops.EPI_SWIGLU, torch.float32)
    assert ops.last_dispatch() == ops.PATH_STREAM
    assert rel_fro(got_auto, got_stream) < 1e-5
    monkeypatch.delenv("NVFP4MOE_FORCE_PATH")
    small = _problem([10, 20, 0, 30], 256, 256, seed=9)
    _run_gemm(small, ops.W4A16, ops.EPI_SWIGLU, torch.float32)
    assert ops.last_dispatch() == ops.PATH_STREAM
    odd = _problem([300, 300], 160, 256, seed=9)                # Nw % 256 != 0: streaming path
    _run_gemm(odd, ops.W4A16, ops.EPI_NONE, torch.float32)
    assert ops.last_dispatch() == ops.PATH_STREAM


# ------------------------------------------------------------------ reduce
@pytest.mark.parametrize("T,k,H,ydt", [(16, 2, 256, torch.float32), (7, 22, 64, torch.bfloat16),
                                       (512, 8, 6144, torch.float32), (300, 8, 7168, torch.bfloat16),
                                       (256, 3, 1000, torch.float32), (260, 2, 8200, torch.float32),
                                       (255, 4, 7168, torch.float32)])
def test_unpermute_reduce(T, k, H, ydt):
    say("reduce", T, k, H, ydt)
    rng = np.random.default_rng(T + k + H)
    y = inputs.random_fp32((T * k, H), T * k).to(ydt)
    s2r = rng.permutation(T * k).astype(np.int32)
    w = rng.random((T, k)).astype(np.float32)
    got = np_(ops.moe_unpermute_reduce(y.to(DEV), torch.from_numpy(s2r).to(DEV), torch.from_numpy(w).to(DEV)))
    assert_finite(got)
    want = assert_reduce_elementwise(got, y.float().numpy(), s2r, w)
    assert rel_fro(got, want) <= W4A16_TOL
