"""NVFP4 format oracle: code tables, unpacking, dequantization, quantization.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``): the product path never
imports this module.

What the pages fix
  * "The Benchmark That Confirmed the Ceiling: NVFP4 Cutlass on sm_120",
    section "The NVFP4 Pivot": NVFP4 is FP4 data with one E4M3 block scale
    per group of 16 elements (as opposed to MXFP4: group 32, UE8M0 scale).
  * Same page, section "Roofline Awareness": an FP4 parameter costs half a
    byte (two values per byte).
  * "Native FP4 Is Slower Than Emulated FP4", section 1: NVFP4 checkpoints
    carry FP4 weights.

Readings taken where the pages are silent:
  * FP4 is E2M1 with the OCP Microscaling (MX) v1.0 bit layout
    (sign, 2 exponent bits with bias 1, 1 mantissa bit); value set
    {0, +-0.5, +-1, +-1.5, +-2, +-3, +-4, +-6}.
  * E4M3 is the OCP FP8 "E4M3FN" variant (bias 7, no infinities, NaN at
    S.1111.111, max 448), which is also gfx950's FP8.
  * Packing: element 2i of a row is the LOW nibble of byte i, element 2i+1
    the HIGH nibble.
  * A matrix additionally carries one FP32 per-tensor ("global") scale g;
    a value decodes as E2M1[q] * E4M3[s] * g.
  * Quantization rule (all float32 steps, round-to-nearest-even):
        amax_T = max |w| over the finite entries of the matrix
        g      = fp32(amax_T / 2688)  (2688 = 6 * 448), or 1 if amax_T == 0
        per 16-group along the row:
          if the group holds a NaN/Inf: scale byte 0x7F (NaN), codes 0
          amax_g == 0               : scale byte 0x00, codes +-0
          else r = min(fp32(amax_g / fp32(6 * g)), 448); s = E4M3_RNE(r)
               S = fp32(E4M3[s] * g)
               q_i = E2M1_RNE_saturating(fp32(w_i / S))   (q_i = +-0 if S == 0)
        The sign bit of every code is the sign bit of its input (-0 -> 0x8).
    A caller may instead supply g (a static scale); then the same per-group
    rule runs with that g.

Parity status: every function below is pinned in tests/test_oracle_nvfp4.py
(closed forms, the OCP value sets, an independent torch float8_e4m3fn cast,
grid-built inputs that must round-trip exactly, exact E2M1 midpoints under
scales that are not powers of two (which only a correctly rounded division
keeps on the midpoint), and error bounds).
"""
from __future__ import annotations

import numpy as np

GROUP = 16               # elements per E4M3 block scale (NVFP4)
E2M1_MAX = 6.0
E4M3_MAX = 448.0
GLOBAL_DENOM = np.float32(E2M1_MAX * E4M3_MAX)  # 2688
E4M3_NAN_CODE = 0x7F


def _e2m1_decode_code(c: int) -> float:
    """Closed form of one E2M1 code (OCP MX FP4): s.ee.m, exponent bias 1."""
    s = (c >> 3) & 1
    e = (c >> 1) & 3
    m = c & 1
    mag = (m * 0.5) if e == 0 else (2.0 ** (e - 1)) * (1.0 + m / 2.0)
    return -mag if s else mag


def _e4m3_decode_code(b: int) -> float:
    """Closed form of one E4M3FN code: s.eeee.mmm, bias 7, NaN at x.1111.111."""
    s = (b >> 7) & 1
    e = (b >> 3) & 15
    m = b & 7
    if e == 15 and m == 7:
        return float("nan")
    if e == 0:
        mag = (m / 8.0) * 2.0 ** -6
    else:
        mag = (1.0 + m / 8.0) * 2.0 ** (e - 7)
    return -mag if s else mag


#: value of each 4-bit code 0..15 (float64)
E2M1_TABLE = np.array([_e2m1_decode_code(c) for c in range(16)], dtype=np.float64)
#: value of each 8-bit E4M3FN code 0..255 (float64, NaN at 0x7F / 0xFF)
E4M3_TABLE = np.array([_e4m3_decode_code(b) for b in range(256)], dtype=np.float64)

# positive grids, ascending; index == code magnitude
_E2M1_POS = E2M1_TABLE[:8].copy()            # codes 0..7
_E4M3_POS = E4M3_TABLE[:0x7F].copy()         # codes 0..0x7E (finite, >= 0)


def _rne_to_grid(x: np.ndarray, grid: np.ndarray) -> np.ndarray:
    """Round non-negative float64 values onto an ascending grid.

    Nearest grid point; an exact midpoint goes to the grid point with the
    even index (even code = mantissa LSB 0). Values above the last grid point
    map to the last index (saturation). Midpoints are few-bit dyadic numbers,
    so the float64 comparisons here are exact.
    """
    x = np.asarray(x, dtype=np.float64)
    hi = np.searchsorted(grid, x, side="left")          # grid[hi-1] < x <= grid[hi]
    hi = np.clip(hi, 0, len(grid) - 1)
    lo = np.clip(hi - 1, 0, len(grid) - 1)
    mid = (grid[lo] + grid[hi]) * 0.5
    out = np.where(x < mid, lo, hi)
    tie = (x == mid) & (lo != hi)
    out = np.where(tie, np.where(lo % 2 == 0, lo, hi), out)
    out = np.where(x >= grid[-1], len(grid) - 1, out)
    out = np.where(x <= 0, 0, out)
    return out.astype(np.uint8)


def e4m3_rne(r: np.ndarray) -> np.ndarray:
    """E4M3FN code (0..0x7E) nearest to each float in [0, 448], ties to even."""
    return _rne_to_grid(r, _E4M3_POS)


def e2m1_rne_sat(x: np.ndarray) -> np.ndarray:
    """E2M1 magnitude code (0..7) nearest to |x|, ties to even, saturating at 6."""
    return _rne_to_grid(np.abs(np.asarray(x, dtype=np.float64)), _E2M1_POS)


def unpack_fp4(packed: np.ndarray) -> np.ndarray:
    """[..., C/2] bytes -> [..., C] 4-bit codes; element 2i = low nibble of byte i."""
    p = np.asarray(packed, dtype=np.uint8)
    out = np.empty(p.shape[:-1] + (p.shape[-1] * 2,), dtype=np.uint8)
    out[..., 0::2] = p & 0x0F
    out[..., 1::2] = p >> 4
    return out


def pack_fp4(codes: np.ndarray) -> np.ndarray:
    """Inverse of :func:`unpack_fp4`."""
    c = np.asarray(codes, dtype=np.uint8)
    assert c.shape[-1] % 2 == 0
    return (c[..., 0::2] & 0x0F) | ((c[..., 1::2] & 0x0F) << 4)


def dequantize(packed: np.ndarray, scales: np.ndarray, g) -> np.ndarray:
    """NVFP4 [R, C] -> float64: E2M1[q] * E4M3[s] * g, s shared by 16 along C.

    ``packed`` is [..., R, C/2] uint8, ``scales`` [..., R, C/16] uint8, ``g`` a
    float32 scalar (or an array broadcastable over the leading batch dims).
    """
    q = unpack_fp4(packed)
    vals = E2M1_TABLE[q]
    sc = E4M3_TABLE[np.asarray(scales, dtype=np.uint8)]
    vals = vals * np.repeat(sc, GROUP, axis=-1)
    g = np.asarray(g, dtype=np.float32).astype(np.float64)
    if g.ndim:
        g = g.reshape(g.shape + (1, 1))
    return vals * g


def div_f32(a, b) -> np.ndarray:
    """Correctly rounded float32 quotient a / b (IEEE division, round to nearest even).

    The quantization rule divides; a reciprocal followed by a multiply rounds twice
    and can move a quotient that is exactly an E2M1 midpoint off it.
    """
    with np.errstate(divide="ignore", invalid="ignore", over="ignore"):
        return (np.asarray(a, dtype=np.float32) / np.asarray(b, dtype=np.float32)).astype(np.float32)


def global_scale(w: np.ndarray) -> np.float32:
    """g = fp32(amax / 2688) over the finite entries; 1.0 when that amax is 0."""
    a = np.abs(np.asarray(w, dtype=np.float32))
    a = a[np.isfinite(a)]
    amax = np.float32(a.max()) if a.size else np.float32(0.0)
    if amax == 0:
        return np.float32(1.0)
    return np.float32(amax / GLOBAL_DENOM)


def quantize(w: np.ndarray, g=None):
    """Quantize one float32 matrix [R, C] (C % 16 == 0) to NVFP4.

    Returns ``(packed [R, C/2] uint8, scales [R, C/16] uint8, g float32)``.
    Follows the rule in the module docstring step by step, in float32 where
    the rule says float32.
    """
    w = np.asarray(w, dtype=np.float32)
    assert w.ndim == 2 and w.shape[1] % GROUP == 0
    R, C = w.shape
    g = global_scale(w) if g is None else np.float32(g)
    grp = w.reshape(R, C // GROUP, GROUP)
    finite = np.isfinite(grp).all(axis=-1)                       # [R, C/16]
    amax_g = np.abs(np.where(np.isfinite(grp), grp, 0)).max(axis=-1).astype(np.float32)
    six_g = np.float32(np.float32(E2M1_MAX) * g)
    ratio = div_f32(amax_g, six_g)                               # fp32 division
    ratio = np.where(amax_g == 0, np.float32(0), ratio)
    ratio = np.minimum(ratio, np.float32(E4M3_MAX))
    s = e4m3_rne(ratio)                                          # [R, C/16]
    S = (E4M3_TABLE[s].astype(np.float32) * g).astype(np.float32)  # fp32 product
    S_el = np.repeat(S, GROUP, axis=-1).reshape(R, C)
    x = div_f32(w, S_el)                                         # fp32 division
    mag = e2m1_rne_sat(np.where(S_el == 0, np.float32(0), x))
    sign = np.signbit(w).astype(np.uint8) << 3
    codes = (mag | sign).astype(np.uint8)
    bad = np.repeat(~finite, GROUP, axis=-1).reshape(R, C)
    codes = np.where(bad, np.uint8(0), codes)
    s = np.where(finite, s, np.uint8(E4M3_NAN_CODE)).astype(np.uint8)
    return pack_fp4(codes), s, np.float32(g)


def quantize_batched(w: np.ndarray, g=None):
    """Quantize B independent matrices [B, R, C], one global scale each."""
    outs = [quantize(w[b], None if g is None else np.asarray(g)[b]) for b in range(w.shape[0])]
    return (np.stack([o[0] for o in outs]), np.stack([o[1] for o in outs]),
            np.array([o[2] for o in outs], dtype=np.float32))
