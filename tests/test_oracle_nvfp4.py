"""Pins of the NVFP4 format oracle against things other than itself (CPU only).

Each test names what it pins the oracle to: a published value set, an
independent library cast (torch.float8_e4m3fn), inputs constructed on the
quantization grid (which must come back unchanged), or a derived error bound.
"""
import math
import os

import numpy as np
import pytest
import torch

from oracle import nvfp4

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _read_table(name):
    rows = []
    for line in open(os.path.join(GOLDEN, name)):
        line = line.strip()
        if not line or line.startswith("#"):
            continue
        a, b = line.split()
        rows.append((a, b))
    return rows


# ------------------------------------------------------------------ E2M1
def test_e2m1_table_matches_ocp_value_set():
    for code, val in _read_table("e2m1_codes.txt"):
        c = int(code, 16)
        v = float(val)
        assert nvfp4.E2M1_TABLE[c] == v
        assert math.copysign(1, nvfp4.E2M1_TABLE[c]) == math.copysign(1, v)
    mags = sorted(set(abs(x) for x in nvfp4.E2M1_TABLE))
    assert mags == [0, 0.5, 1, 1.5, 2, 3, 4, 6]


def test_e2m1_rne_ties_and_saturation():
    for x, code in _read_table("e2m1_rne_ties.txt"):
        xv = np.float32(float(x))
        assert int(nvfp4.e2m1_rne_sat(np.array([xv]))[0]) == int(code, 16), x
        assert int(nvfp4.e2m1_rne_sat(np.array([-xv]))[0]) == int(code, 16), x


def test_e2m1_rne_is_nearest_by_exhaustive_distance():
    rng = np.random.default_rng(1)
    x = np.concatenate([rng.uniform(0, 7, 20000), rng.uniform(0, 1, 5000)]).astype(np.float32)
    got = nvfp4.e2m1_rne_sat(x)
    grid = nvfp4.E2M1_TABLE[:8]
    d = np.abs(x.astype(np.float64)[:, None] - grid[None, :])
    best = d.min(axis=1)
    assert np.all(d[np.arange(len(x)), got] == best)


# ------------------------------------------------------------------ E4M3
def test_e4m3_table_matches_torch_float8_e4m3fn_all_codes():
    ref = torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn).double().numpy()
    ours = nvfp4.E4M3_TABLE
    nan = np.isnan(ref)
    assert np.array_equal(nan, np.isnan(ours))
    assert np.array_equal(ref[~nan], ours[~nan])
    assert np.array_equal(np.signbit(ref[~nan]), np.signbit(ours[~nan]))
    assert list(np.nonzero(nan)[0]) == [0x7F, 0xFF]


def test_e4m3_landmarks():
    for code, val in _read_table("e4m3_special.txt"):
        c = int(code, 16)
        if val == "nan":
            assert np.isnan(nvfp4.E4M3_TABLE[c])
        else:
            assert nvfp4.E4M3_TABLE[c] == float(val)


def _torch_e4m3(x32):
    return torch.from_numpy(np.asarray(x32, np.float32)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def test_e4m3_rne_matches_torch_cast():
    pos = nvfp4.E4M3_TABLE[:0x7F]
    mids = (pos[:-1] + pos[1:]) / 2
    rng = np.random.default_rng(2)
    x = np.concatenate([
        pos, mids, np.nextafter(mids.astype(np.float32), 0), np.nextafter(mids.astype(np.float32), 1000),
        np.exp2(rng.uniform(-12, np.log2(448), 50000)),
        rng.uniform(0, 2.0 ** -6, 5000),
    ]).astype(np.float32)
    x = x[(x >= 0) & (x <= 448)]
    assert np.array_equal(nvfp4.e4m3_rne(x), _torch_e4m3(x))


# ------------------------------------------------------------- packing
def test_pack_low_nibble_first():
    codes = np.array([[1, 2, 3, 4, 0xF, 0x8]], dtype=np.uint8)
    p = nvfp4.pack_fp4(codes)
    assert p.tolist() == [[0x21, 0x43, 0x8F]]
    assert np.array_equal(nvfp4.unpack_fp4(p), codes)


def test_dequantize_hand_example():
    codes = np.arange(32, dtype=np.uint8).reshape(1, 32) % 16
    packed = nvfp4.pack_fp4(codes)
    scales = np.array([[0x38, 0x39]], dtype=np.uint8)   # 1.0 and 1.125
    g = np.float32(2.0)
    want = np.concatenate([nvfp4.E2M1_TABLE * 1.0 * 2, nvfp4.E2M1_TABLE * 1.125 * 2])
    got = nvfp4.dequantize(packed, scales, g)[0]
    assert np.array_equal(got, want)


# ------------------------------------------------------------- quantize
def _grid_matrix(rng, R, C, g, force_top=True):
    """w = E2M1[q] * E4M3[s] * g with g a power of two (every product exact in fp32)."""
    G = C // 16
    s = rng.integers(0x10, 0x7E, size=(R, G)).astype(np.uint8)
    q = rng.integers(0, 16, size=(R, C)).astype(np.uint8)
    q = q.reshape(R, G, 16)
    q[:, :, 0] = np.where(rng.random((R, G)) < 0.5, 0x7, 0xF)     # a +-6 in every group
    q = q.reshape(R, C)
    if force_top:
        s[0, 0] = 0x7E                                              # amax = 6 * 448 * g
    w = (nvfp4.E2M1_TABLE[q] * np.repeat(nvfp4.E4M3_TABLE[s], 16, axis=1) * float(g)).astype(np.float32)
    return w, q, s


@pytest.mark.parametrize("g", [2.0 ** -7, 1.0, 2.0 ** 5])
def test_quantize_grid_inputs_roundtrip_exactly_static_g(g):
    rng = np.random.default_rng(3)
    w, q, s = _grid_matrix(rng, 24, 128, g, force_top=False)
    packed, scales, gg = nvfp4.quantize(w, g=np.float32(g))
    assert gg == np.float32(g)
    assert np.array_equal(scales, s)
    assert np.array_equal(nvfp4.unpack_fp4(packed), q)


def test_quantize_grid_inputs_roundtrip_exactly_dynamic_g():
    rng = np.random.default_rng(4)
    g = np.float32(2.0 ** -9)
    w, q, s = _grid_matrix(rng, 16, 256, g)
    packed, scales, gg = nvfp4.quantize(w)
    assert gg == g                       # amax / 2688 = 6 * 448 * g / 2688
    assert np.array_equal(scales, s)
    assert np.array_equal(nvfp4.unpack_fp4(packed), q)


MIDPOINTS = ("0.25", "0.75", "1.25", "1.75", "2.5", "3.5", "5.0")


def tie_matrix(g):
    """Rows of exact E2M1 midpoints under scales S = E4M3[s] * g that are not powers of two.

    Row i uses scale code s = 8 + i (every normal code up to 0x7E): element 0 is 6 S, which
    makes 6 S / (6 g) = E4M3[s] exactly and so fixes the scale code; elements 1..7 are m S and
    8..14 are -m S for the seven midpoints m; element 15 is 0. With g = 3, 5 or 7 times a power
    of two every product has at most 10 significant bits, so each input is exact in float32 and
    a correctly rounded division returns m itself. Returns (w [118, 16] float32, the scale
    codes, the expected 4-bit codes from the hand-derived tie table).
    """
    ties = {x: int(c, 16) for x, c in _read_table("e2m1_rne_ties.txt") if x in MIDPOINTS}
    mids = [float(m) for m in MIDPOINTS]
    s_codes = np.arange(8, 0x7F, dtype=np.uint8)
    rows, want = [], []
    for s in s_codes:
        S = nvfp4.E4M3_TABLE[s] * float(g)
        rows.append([6 * S] + [m * S for m in mids] + [-m * S for m in mids] + [0.0])
        want.append([0x7] + [ties[m] for m in MIDPOINTS] + [0x8 | ties[m] for m in MIDPOINTS] + [0x0])
    w = np.array(rows, dtype=np.float64)
    assert np.array_equal(w.astype(np.float32).astype(np.float64), w)   # exact in float32
    return w.astype(np.float32), s_codes[:, None], np.array(want, dtype=np.uint8)


@pytest.mark.parametrize("g", [3 * 2.0 ** -10, 5 * 2.0 ** -12, 7 * 2.0 ** -9])
def test_quantize_exact_midpoints_divide_correctly(g):
    """Pinned to the tie table: a quotient that is exactly an E2M1 midpoint goes to the even
    code. A reciprocal-then-multiply (two roundings) moves some of these quotients off the
    midpoint and picks the odd neighbour."""
    w, s_want, q_want = tie_matrix(g)
    packed, scales, gg = nvfp4.quantize(w, g=np.float32(g))
    assert gg == np.float32(g)
    assert np.array_equal(scales, s_want)
    assert np.array_equal(nvfp4.unpack_fp4(packed), q_want)


def test_quantize_scale_codes_match_torch_cast_of_ratio():
    rng = np.random.default_rng(5)
    w = (rng.standard_normal((64, 512)) * 0.02).astype(np.float32)
    w[3, :16] *= 1e-6                     # tiny groups -> subnormal scale codes
    packed, scales, g = nvfp4.quantize(w)
    amax_g = np.abs(w.reshape(64, 32, 16)).max(-1).astype(np.float32)
    ratio = np.minimum((amax_g / np.float32(np.float32(6) * g)).astype(np.float32), np.float32(448))
    assert np.array_equal(scales, _torch_e4m3(ratio))
    assert g == np.float32(np.abs(w).max() / np.float32(2688))


def test_quantize_group_amax_maps_to_six():
    rng = np.random.default_rng(6)
    w = (rng.standard_normal((32, 1024)) * 0.02).astype(np.float32)
    packed, scales, g = nvfp4.quantize(w)
    q = nvfp4.unpack_fp4(packed).reshape(32, 64, 16)
    idx = np.abs(w.reshape(32, 64, 16)).argmax(-1)
    top = np.take_along_axis(q, idx[..., None], -1)[..., 0]
    normal = scales >= 0x08
    assert normal.all()
    assert np.all((top[normal] & 7) == 7)


def test_quantize_error_bound_per_element():
    rng = np.random.default_rng(7)
    w = (rng.standard_normal((48, 768)) * 0.02).astype(np.float32)
    w[0, :32] = rng.standard_normal(32) * 1e-5
    packed, scales, g = nvfp4.quantize(w)
    wh = nvfp4.dequantize(packed, scales, g)
    S = np.repeat(nvfp4.E4M3_TABLE[scales] * float(g), 16, axis=1)
    x = np.abs(w.astype(np.float64)) / S
    half_step = np.where(x <= 2, 0.25, np.where(x <= 4, 0.5, 1.0))
    bound = S * np.maximum(half_step, x - 6) + np.abs(w) * 2.0 ** -22
    assert np.all(np.abs(w - wh) <= bound)


def test_quantize_gaussian_error_level():
    rng = np.random.default_rng(8)
    w = (rng.standard_normal((256, 2048)) * 0.02).astype(np.float32)
    packed, scales, g = nvfp4.quantize(w)
    wh = nvfp4.dequantize(packed, scales, g)
    rel = np.linalg.norm(w - wh) / np.linalg.norm(w)
    assert 0.08 < rel < 0.11                         # statistical guard, not a spec


def test_quantize_nonfinite_and_zero_groups():
    w = np.zeros((2, 64), dtype=np.float32)
    w[0, 16:32] = np.linspace(-1, 1, 16)
    w[0, 20] = np.nan
    w[1, 40] = np.inf
    w[1, 48:64] = 3.0
    w[1, 0] = -0.0
    packed, scales, g = nvfp4.quantize(w)
    assert g == np.float32(np.float32(3.0) / np.float32(2688))
    assert scales[0, 1] == 0x7F and scales[1, 2] == 0x7F
    q = nvfp4.unpack_fp4(packed)
    assert np.all(q[0, 16:32] == 0) and np.all(q[1, 32:48] == 0)
    assert scales[0, 0] == 0 and scales[0, 2] == 0 and scales[1, 0] == 0
    assert q[1, 0] == 0x8                            # -0 keeps its sign bit
    assert np.all(q[1, 48:64] == 0x7) and scales[1, 3] == 0x7E
    dq = nvfp4.dequantize(packed, scales, g)
    assert np.all(np.isnan(dq[0, 16:32])) and np.all(np.isnan(dq[1, 32:48]))


def test_quantize_all_zero_matrix():
    packed, scales, g = nvfp4.quantize(np.zeros((4, 32), np.float32))
    assert g == 1.0 and not scales.any() and not packed.any()


def test_quantize_static_scale_saturates():
    w = np.full((1, 16), 100.0, dtype=np.float32)
    packed, scales, g = nvfp4.quantize(w, g=np.float32(1e-3))   # ratio 1.7e4 > 448
    assert scales[0, 0] == 0x7E
    assert np.all(nvfp4.unpack_fp4(packed) == 0x7)
