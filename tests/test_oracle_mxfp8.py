"""Pins of the MXFP8 (block-scaled FP8) format oracle against things other than itself (CPU only).

Element codes against an independent library cast (torch.float8_e4m3fn of the scaled,
clamped float32 values), scale bytes against the floor(log2) closed form, inputs built on
the quantization grid (which must come back unchanged), the largest-code invariant of the
shared-exponent rule, a derived element error bound, and special groups.
"""
import math

import numpy as np
import pytest
import torch

from oracle import mxfp4, mxfp8, nvfp4


def test_codes_match_torch_e4m3fn_cast():
    rng = np.random.default_rng(21)
    w = (rng.standard_normal((48, 256)) * np.exp(rng.uniform(-12, 12, (48, 1)))).astype(np.float32)
    w[0, :32] = 0.0
    w[0, 5] = -0.0
    c, s = mxfp8.quantize(w)
    amax = np.abs(w.reshape(48, 8, 32)).max(axis=-1)
    e = np.where(amax > 0, np.floor(np.log2(amax.astype(np.float64))) - 8, 0).astype(np.int64)
    e = np.maximum(e, -127)
    assert np.array_equal(s.astype(np.int64), np.where(amax > 0, e + 127, 0))
    x = np.ldexp(w.astype(np.float64), -np.repeat(e, 32, axis=1)).astype(np.float32)
    ref = torch.from_numpy(np.clip(x, -448, 448)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(c, ref)


def _grid(rng, R, C):
    """E4M3[code] * 2^e with, in every 32-group, one element of magnitude in [256, 448]
    (codes 0x78..0x7E), so floor(log2 amax) = e + 8 and the rule must return the codes."""
    codes = rng.integers(0, 0x7F, size=(R, C)).astype(np.uint8) | (rng.integers(0, 2, size=(R, C)) << 7).astype(np.uint8)
    G = C // 32
    e = rng.integers(-100, 100, size=(R, G))
    lead = rng.integers(0, 32, size=(R, G))
    for r in range(R):
        for g in range(G):
            codes[r, 32 * g + lead[r, g]] = (rng.integers(0, 2) << 7) | rng.integers(0x78, 0x7F)
    vals = nvfp4.E4M3_TABLE[codes] * np.ldexp(1.0, np.repeat(e, 32, axis=1))
    return codes, e, vals.astype(np.float32)


def test_grid_inputs_round_trip_exactly():
    rng = np.random.default_rng(22)
    codes, e, w = _grid(rng, 16, 256)
    c, s = mxfp8.quantize(w)
    assert np.array_equal(c, codes)
    assert np.array_equal(s.astype(np.int64), e + 127)
    assert np.array_equal(mxfp8.dequantize(c, s), w.astype(np.float64))


def test_largest_code_in_top_binade():
    rng = np.random.default_rng(23)
    w = (rng.standard_normal((64, 512)) * np.exp(rng.uniform(-20, 20, (64, 1)))).astype(np.float32)
    c, _ = mxfp8.quantize(w)
    top = (c & 0x7F).reshape(64, 16, 32).max(axis=-1)
    assert ((top >= 0x78) & (top <= 0x7E)).all()


def test_element_error_bound():
    """|w - w^| <= 2^e * (half an E4M3 step at |w| 2^-e, or the saturation excess)."""
    rng = np.random.default_rng(24)
    w = (rng.standard_normal((32, 1024)) * 3).astype(np.float32)
    c, s = mxfp8.quantize(w)
    d = mxfp8.dequantize(c, s)
    e = np.repeat(s.astype(np.int64) - 127, 32, axis=1)
    x = np.abs(w.astype(np.float64)) * np.ldexp(1.0, -e)
    # E4M3 step at x: 2^(floor(log2 x) - 3) for normals (x >= 2^-6), 2^-9 below
    step = np.where(x >= 2.0 ** -6, np.ldexp(1.0, np.floor(np.log2(np.maximum(x, 2.0 ** -6))).astype(np.int64) - 3),
                    2.0 ** -9)
    bound = np.ldexp(np.where(x <= 448, step / 2, x - 448), e)
    assert (np.abs(w - d) <= bound).all()
    assert (x < 512).all()


def test_special_groups():
    w = np.zeros((4, 32), np.float32)
    w[1, 3] = np.nan
    w[2, 0] = -np.inf
    w[3, :] = -0.0
    c, s = mxfp8.quantize(w)
    assert s[:, 0].tolist() == [0, 255, 255, 0]
    assert (c[0] == 0).all() and (c[1] == 0).all() and (c[2] == 0).all() and (c[3] == 0x80).all()
    t = np.full((1, 32), 2.0 ** -150, np.float32)      # far below the smallest scale: rounds to 0
    c, s = mxfp8.quantize(t)
    assert s[0, 0] == 0 and (c == 0).all()


def test_hand_example():
    w = np.zeros((1, 32), np.float32)
    w[0, 0] = 1.0        # amax 1: e = -8, 1 * 2^8 = 256 -> code 0x78
    w[0, 1] = -0.5       # -128 -> 0x80 | 0x70
    w[0, 2] = 1.0 + 1 / 16   # 272: between 256 and 288 (step 32), a tie -> even code 0x78
    c, s = mxfp8.quantize(w)
    assert s[0, 0] == 127 - 8
    assert c[0, 0] == 0x78 and c[0, 1] == 0xF0 and c[0, 2] == 0x78
    assert mxfp8.dequantize(c, s)[0, 1] == -0.5


@pytest.mark.parametrize("x", [1.0, 300.0, 511.9, 2.0 ** -126, 3.4e38])
def test_shared_exponent_closed_form(x):
    e = int(mxfp8.shared_exponent(np.float32(x)))
    assert e == max(math.floor(math.log2(float(np.float32(x)))) - 8, -127)


def test_scale_table_is_the_mx_one():
    assert mxfp8.dequantize(np.array([[0x38] * 32], np.uint8), np.array([[127]], np.uint8))[0, 0] == 1.0
    assert np.isnan(mxfp4.E8M0_TABLE[255])
