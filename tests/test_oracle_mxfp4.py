"""Pins of the MXFP4 format oracle against things other than itself (CPU only).

Each test names what it pins the oracle to: an independent library cast
(torch.float8_e8m0fnu for the UE8M0 scale), inputs constructed on the
quantization grid (which must come back unchanged), the largest-code invariant
of the shared-exponent rule, a derived element error bound, and hand examples.
"""
import math

import numpy as np
import pytest
import torch

from oracle import mxfp4, nvfp4


# ------------------------------------------------------------------ UE8M0
def test_e8m0_table_matches_torch_cast():
    ref = torch.arange(256, dtype=torch.int32).to(torch.uint8).view(torch.float8_e8m0fnu).double().numpy()
    assert np.isnan(mxfp4.E8M0_TABLE[255]) and np.isnan(ref[255])
    assert np.array_equal(mxfp4.E8M0_TABLE[:255], ref[:255])
    assert mxfp4.E8M0_TABLE[127] == 1.0 and mxfp4.E8M0_TABLE[0] == 2.0 ** -127 and mxfp4.E8M0_TABLE[254] == 2.0 ** 127


# ------------------------------------------------------------------ hand examples
def test_hand_examples():
    w = np.zeros((1, 64), np.float32)
    w[0, 0] = 1.0                 # amax 1: e = 0 - 2, 1 * 2^2 = 4 -> code 6 (magnitude 4)
    w[0, 1] = -0.25               # -0.25 * 4 = -1 -> code 0x8 | 2
    w[0, 32] = 7.0                # amax 7: e = 2 - 2 = 0, 7 saturates to 6 (code 7)
    w[0, 33] = 2.5                # 2.5: tie between 2 (code 4) and 3 (code 5) -> even code 4
    p, s = mxfp4.quantize(w)
    c = nvfp4.unpack_fp4(p)[0]
    assert s.tolist() == [[125, 127]]
    assert c[0] == 6 and c[1] == (0x8 | 2) and c[2] == 0
    assert c[32] == 7 and c[33] == 4
    d = mxfp4.dequantize(p, s)[0]
    assert d[0] == 1.0 and d[1] == -0.25 and d[32] == 6.0 and d[33] == 2.0


# ------------------------------------------------------------------ quantize
def _grid_matrix(rng, R, C):
    """Values E2M1[code] * 2^e with, in every 32-group, one element of magnitude
    4 or 6 (so floor(log2 amax) = e + 2 and the rule must return the codes)."""
    codes = rng.integers(0, 16, size=(R, C)).astype(np.uint8)
    G = C // 32
    e = rng.integers(-100, 100, size=(R, G))
    lead = rng.integers(0, 32, size=(R, G))
    for r in range(R):
        for g in range(G):
            codes[r, 32 * g + lead[r, g]] = (rng.integers(0, 2) << 3) | rng.choice([6, 7])
    vals = nvfp4.E2M1_TABLE[codes] * np.ldexp(1.0, np.repeat(e, 32, axis=1))
    return codes, e, vals.astype(np.float32)


def test_grid_inputs_round_trip_exactly():
    rng = np.random.default_rng(11)
    codes, e, w = _grid_matrix(rng, 24, 256)
    p, s = mxfp4.quantize(w)
    got = nvfp4.unpack_fp4(p)
    # -0 inputs keep their sign bit: code 0x8 stays 0x8
    assert np.array_equal(got, codes)
    assert np.array_equal(s.astype(np.int64), e + 127)
    assert np.array_equal(mxfp4.dequantize(p, s), w.astype(np.float64))


def test_largest_code_is_4_or_6():
    rng = np.random.default_rng(12)
    w = (rng.standard_normal((64, 512)) * np.exp(rng.uniform(-20, 20, (64, 1)))).astype(np.float32)
    p, s = mxfp4.quantize(w)
    mags = nvfp4.unpack_fp4(p).reshape(64, 16, 32) & 7
    assert np.isin(mags.max(axis=-1), [6, 7]).all()


def test_element_error_bound():
    """|w - w^| <= 2^e * (half the E2M1 step at |w| 2^-e, or the saturation excess)."""
    rng = np.random.default_rng(13)
    w = (rng.standard_normal((32, 1024)) * 3).astype(np.float32)
    p, s = mxfp4.quantize(w)
    d = mxfp4.dequantize(p, s)
    e = np.repeat(s.astype(np.int64) - 127, 32, axis=1)
    x = np.abs(w.astype(np.float64)) * np.ldexp(1.0, -e)
    half = np.where(x < 2, 0.25, np.where(x < 4, 0.5, 1.0))
    bound = np.ldexp(np.where(x <= 6, half, x - 6), e)
    assert (np.abs(w - d) <= bound).all()
    assert (x < 8).all()


def test_special_groups():
    w = np.zeros((4, 32), np.float32)
    w[1, 3] = np.nan
    w[2, 0] = np.inf
    w[3, :] = -0.0
    p, s = mxfp4.quantize(w)
    c = nvfp4.unpack_fp4(p)
    assert s[:, 0].tolist() == [0, 255, 255, 0]
    assert (c[0] == 0).all() and (c[1] == 0).all() and (c[2] == 0).all() and (c[3] == 8).all()
    # a group far below the smallest scale: e clamps at -127 and the values round to 0
    t = np.full((1, 32), 2.0 ** -130, np.float32)
    p, s = mxfp4.quantize(t)
    assert s[0, 0] == 0 and (nvfp4.unpack_fp4(p) == 0).all()


@pytest.mark.parametrize("x", [1.0, 1.5, 3.9999998, 4.0, 2.0 ** -126, 2.0 ** -140, 3.4e38])
def test_shared_exponent_closed_form(x):
    e = int(mxfp4.shared_exponent(np.float32(x)))
    assert e == max(math.floor(math.log2(float(np.float32(x)))) - 2, -127)
