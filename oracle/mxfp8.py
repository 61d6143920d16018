"""MXFP8 format oracle: FP8 E4M3 elements with one UE8M0 scale per 32.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``): the product path never
imports this module.

What the pages fix
  * "Native FP4 Is Slower Than Emulated FP4", sections 1 and 2: the model runs
    FP8 activations, and its dense layers go through FP8 scaled-matmul kernels;
    the kernels named there are scaled with a per-tensor or a per-channel
    scale. None of them is block-scaled.
  * "The Benchmark That Confirmed the Ceiling", section "The NVFP4 Pivot": the
    MX family's shared scale is UE8M0 per group of 32.

Readings taken where the pages are silent:
  * The block-scaled FP8 dense GEMM is a reading, not something the pages
    name: it applies the pages' MX-family scale (UE8M0 per 32) to the FP8
    elements of their dense layers.
  * Block-scaled FP8 is the OCP MX v1.0 MXFP8 (E4M3) format: element codes are
    OCP E4M3FN (the table and rounding of ``oracle/nvfp4.py``), one UE8M0 scale
    2^(s - 127) per 32 consecutive elements of a row (``oracle/mxfp4.py``).
  * Quantization follows the MX v1.0 conversion rule per 32-group, in float32:
        if the group holds a NaN/Inf: scale byte 0xFF (NaN), codes 0
        amax == 0                   : scale byte 0 (2^-127), codes +-0
        else e = floor(log2(amax)) - 8      (8 = the largest E4M3 exponent)
             e = max(e, -127)
             q_i = E4M3_RNE(min(|w_i| * 2^-e, 448)) with the sign bit of w_i
    so amax * 2^-e lies in [256, 512): the group's largest code is 0x78..0x7E
    (values in (448, 512) * 2^e saturate to 448).

Parity status: every function below is pinned in tests/test_oracle_mxfp8.py
(element codes against an independent torch float8_e4m3fn cast, grid-built
inputs that must round-trip exactly, the largest-code invariant, the element
error bound and special groups).
"""
from __future__ import annotations

import numpy as np

from . import mxfp4, nvfp4

GROUP = 32
E4M3_EMAX = 8            # 448 = 1.75 * 2^8
E8M0_NAN_CODE = 0xFF


def dequantize(codes: np.ndarray, scales: np.ndarray) -> np.ndarray:
    """MXFP8 [..., R, C] -> float64: E4M3[q] * 2^(s - 127), s shared by 32 along C.

    ``codes`` is [..., R, C] uint8 (one E4M3 code per element), ``scales``
    [..., R, C/32] uint8.
    """
    vals = nvfp4.E4M3_TABLE[np.asarray(codes, dtype=np.uint8)]
    sc = mxfp4.E8M0_TABLE[np.asarray(scales, dtype=np.uint8)]
    return vals * np.repeat(sc, GROUP, axis=-1)


def shared_exponent(amax: np.ndarray) -> np.ndarray:
    """e = max(floor(log2(amax)) - 8, -127) for finite amax > 0 (float32 input);
    floor(log2) is read off the float32 exponent exactly."""
    a = np.asarray(amax, dtype=np.float32)
    _, x = np.frexp(a)
    return np.maximum(x.astype(np.int64) - 1 - E4M3_EMAX, -127)


def quantize(w: np.ndarray):
    """Quantize one float32 matrix [R, C] (C % 32 == 0) to MXFP8.

    Returns ``(codes [R, C] uint8, scales [R, C/32] uint8)`` by the rule in the
    module docstring, step by step.
    """
    w = np.asarray(w, dtype=np.float32)
    assert w.ndim == 2 and w.shape[1] % GROUP == 0
    R, C = w.shape
    grp = w.reshape(R, C // GROUP, GROUP)
    finite = np.isfinite(grp).all(axis=-1)
    amax = np.abs(np.where(np.isfinite(grp), grp, 0)).max(axis=-1).astype(np.float32)
    e = shared_exponent(np.where(amax > 0, amax, np.float32(1)))
    s = np.where(amax > 0, e + 127, 0)
    s = np.where(finite, s, E8M0_NAN_CODE).astype(np.uint8)
    e_el = np.repeat(np.where(amax > 0, e, 0), GROUP, axis=1)
    # |w| * 2^-e is exact in float64 (a power-of-two scaling of a float32)
    x = np.ldexp(np.abs(w.astype(np.float64)), -e_el)
    x = np.where(np.isfinite(x), x, 0.0)
    mag = nvfp4.e4m3_rne(np.minimum(x, nvfp4.E4M3_MAX))
    mag = np.where(np.repeat(amax > 0, GROUP, axis=1), mag, 0).astype(np.uint8)
    codes = (mag | (np.signbit(w).astype(np.uint8) << 7)).astype(np.uint8)
    codes = np.where(np.repeat(~finite, GROUP, axis=1), np.uint8(0), codes)
    return codes, s


def quantize_batched(w: np.ndarray):
    """Quantize B independent matrices [B, R, C]."""
    outs = [quantize(w[b]) for b in range(w.shape[0])]
    return np.stack([o[0] for o in outs]), np.stack([o[1] for o in outs])
