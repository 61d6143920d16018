"""MXFP4 format oracle: E8M0 scale codes, dequantization, quantization.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``): the product path never
imports this module.

What the pages fix
  * "The Benchmark That Confirmed the Ceiling: NVFP4 Cutlass on sm_120",
    section "The NVFP4 Pivot": MXFP4 is FP4 data with one UE8M0 scale per
    group of 32 elements (the format NVFP4, group 16 with E4M3 scales, is
    contrasted with).

Readings taken where the pages are silent:
  * FP4 codes, their packing (element 2i in the LOW nibble of byte i) and the
    E2M1 value set are those of the NVFP4 oracle (``oracle/nvfp4.py``).
  * UE8M0 is the OCP Microscaling (MX) v1.0 shared-scale format: an unsigned
    8-bit biased exponent, value 2^(s - 127) for s = 0..254, NaN for s = 255.
    There is no per-tensor scale: a value decodes as E2M1[q] * 2^(s - 127).
  * Quantization follows the MX v1.0 conversion rule, per 32-group along the
    row, in float32:
        if the group holds a NaN/Inf: scale byte 0xFF (NaN), codes 0
        amax == 0                   : scale byte 0 (2^-127), codes +-0
        else e = floor(log2(amax)) - 2      (2 = the largest E2M1 exponent)
             e = max(e, -127)               (the smallest UE8M0 scale)
             s = e + 127
             q_i = E2M1_RNE_saturating(w_i * 2^-e)   (exact: a power of two)
    so amax * 2^-e lies in [4, 8) and the group's largest code is 4 or 6
    (values in (6, 8) * 2^e saturate to 6). The sign bit of every code is the
    sign bit of its input.

Parity status: every function below is pinned in tests/test_oracle_mxfp4.py
(the UE8M0 closed form against an independent torch float8_e8m0fnu cast,
grid-built inputs that must round-trip exactly, the largest-code invariant
and the element error bound).
"""
from __future__ import annotations

import math

import numpy as np

from . import nvfp4

GROUP = 32               # elements per UE8M0 scale (MXFP4)
E8M0_NAN_CODE = 0xFF
E2M1_EMAX = 2            # 6 = 1.5 * 2^2


def _e8m0_decode_code(s: int) -> float:
    """Closed form of one UE8M0 code: 2^(s - 127), NaN at 0xFF."""
    return float("nan") if s == E8M0_NAN_CODE else math.ldexp(1.0, s - 127)


#: value of each 8-bit UE8M0 code 0..255 (float64, NaN at 0xFF)
E8M0_TABLE = np.array([_e8m0_decode_code(s) for s in range(256)], dtype=np.float64)


def dequantize(packed: np.ndarray, scales: np.ndarray) -> np.ndarray:
    """MXFP4 [..., R, C] -> float64: E2M1[q] * 2^(s - 127), s shared by 32 along C.

    ``packed`` is [..., R, C/2] uint8, ``scales`` [..., R, C/32] uint8.
    """
    q = nvfp4.unpack_fp4(packed)
    vals = nvfp4.E2M1_TABLE[q]
    sc = E8M0_TABLE[np.asarray(scales, dtype=np.uint8)]
    return vals * np.repeat(sc, GROUP, axis=-1)


def shared_exponent(amax: np.ndarray) -> np.ndarray:
    """e = max(floor(log2(amax)) - 2, -127) for finite amax > 0 (float32 input).

    floor(log2(a)) is read off the float32 exponent exactly (frexp gives
    a = f * 2^x with f in [0.5, 1), so floor(log2(a)) = x - 1), subnormals
    included.
    """
    a = np.asarray(amax, dtype=np.float32)
    _, x = np.frexp(a)
    return np.maximum(x.astype(np.int64) - 1 - E2M1_EMAX, -127)


def quantize(w: np.ndarray):
    """Quantize one float32 matrix [R, C] (C % 32 == 0) to MXFP4.

    Returns ``(packed [R, C/2] uint8, scales [R, C/32] uint8)``, following the
    rule in the module docstring step by step.
    """
    w = np.asarray(w, dtype=np.float32)
    assert w.ndim == 2 and w.shape[1] % GROUP == 0
    R, C = w.shape
    grp = w.reshape(R, C // GROUP, GROUP)
    finite = np.isfinite(grp).all(axis=-1)                          # [R, C/32]
    amax = np.abs(np.where(np.isfinite(grp), grp, 0)).max(axis=-1).astype(np.float32)
    e = shared_exponent(np.where(amax > 0, amax, np.float32(1)))    # [R, C/32]
    s = np.where(amax > 0, e + 127, 0)
    s = np.where(finite, s, E8M0_NAN_CODE).astype(np.uint8)
    # w * 2^-e is exact in float64 (and equals the float32 product: a power of two)
    e_el = np.repeat(np.where(amax > 0, e, 0), GROUP, axis=-1).reshape(R, C)
    x = np.ldexp(w.astype(np.float64), -e_el)
    mag = nvfp4.e2m1_rne_sat(np.where(np.repeat(amax > 0, GROUP, axis=-1).reshape(R, C), x, 0.0))
    sign = np.signbit(w).astype(np.uint8) << 3
    codes = (mag | sign).astype(np.uint8)
    bad = np.repeat(~finite, GROUP, axis=-1).reshape(R, C)
    codes = np.where(bad, np.uint8(0), codes)
    return nvfp4.pack_fp4(codes), s


def quantize_batched(w: np.ndarray):
    """Quantize B independent matrices [B, R, C]."""
    outs = [quantize(w[b]) for b in range(w.shape[0])]
    return np.stack([o[0] for o in outs]), np.stack([o[1] for o in outs])
