"""MoE layer oracle: route -> permute -> up/gate GEMM + SwiGLU -> down GEMM -> reduce.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``): the product path never
imports this module.

What the pages fix
  * "The 2x Gap: Diagnosing Suboptimal FP4 GEMM Kernels on Blackwell SM120",
    sections "The Investigation So Far" and "Discovering the sgl_kernel
    Alternative": tokens are routed top-k (8 of 256 experts) and each expert
    multiplies its tokens by FP4 weights with per-block scales and an alpha;
    a fused MoE gathers tokens to experts and scatters results back.
  * "Native FP4 Is Slower Than Emulated FP4", section 1: 512 experts, 22 active
    per token; "FP4 weights with FP8 activations".
  * "The 24% Ceiling", sections "The Core Insight" and "The Decision":
    W4A16 (FP4 weights dequantized to BF16, BF16 products) versus W4A4
    (FP4 x FP4 products).

Readings taken where the pages are silent:
  * Router: softmax over the E logits, keep the k largest (ranked by logit in
    float32, ties to the lower expert id), renormalise the kept
    probabilities to sum to one.
  * Permutation: stable counting sort of the T*k slots (slot s = t*k + j) by
    expert id; rows of one expert keep ascending slot order.
  * Expert MLP: W13_e = [2F, H] with gate rows 0..F-1 and up rows F..2F-1,
    W2_e = [H, F]; h = silu(gate) * up with silu(x) = x / (1 + e^-x);
    no bias, no clamp.
  * Rounding points: h is rounded to bf16 (W4A16) or NVFP4-quantized with a
    dynamic per-tensor scale (W4A4); router weights are applied in the final
    weighted sum; the layer output is rounded to bf16 once.
  * W4A4 activations: each token row is NVFP4-quantized by the same rule as
    the weights, with one dynamic global scale per activation tensor.
  * FP8 activations: x -> E4M3 with a per-tensor scale amax/448, then back to
    bf16.
  * MXFP4 layer ("The Benchmark That Confirmed the Ceiling", section "The
    NVFP4 Pivot", names MXFP4 as the group-32 UE8M0 alternative): weights,
    token activations and h are all MXFP4 (rule in ``oracle/mxfp4.py``);
    there is no per-tensor scale, so h needs no amax pass.

Parity status: every function is pinned in tests/test_oracle_moe.py
(brute-force sorting, library argsort, exact rational arithmetic on tiny
shapes, closed forms of silu, reduction to a dense FFN computed by torch in
each mode: W4A16, NVFP4 W4A4 with x and h quantized as whole tensors, and
MXFP4).
"""
from __future__ import annotations

import numpy as np

from . import mxfp4, nvfp4


# ----------------------------------------------------------------- roundings
def bf16_round(x: np.ndarray) -> np.ndarray:
    """Round float64 values to the nearest bfloat16 (ties to even), returned as float64.

    bfloat16 keeps 8 significant bits with float32's exponent range
    (normals down to 2^-126, subnormal quantum 2^-133); out-of-range
    magnitudes become +-inf. Rounds once, directly from the float64 value.
    """
    x = np.asarray(x, dtype=np.float64)
    out = np.array(x, copy=True)
    fin = np.isfinite(x) & (x != 0)
    xf = x[fin]
    m, e = np.frexp(xf)                      # xf = m * 2^e, 0.5 <= |m| < 1
    q = np.ldexp(np.rint(np.ldexp(m, 8)), e - 8)   # 8 significant bits
    sub = e < -125                           # below the normal range of bf16
    q[sub] = np.ldexp(np.rint(np.ldexp(xf[sub], 133)), -133)
    big = np.abs(q) > float(np.ldexp(255.0, 120))  # > max bf16 = (2 - 2^-7) * 2^127
    q[big] = np.copysign(np.inf, xf[big])
    out[fin] = q
    return out


def fp32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """bf16 bit patterns (uint16) of float32 data rounded to nearest even (finite inputs)."""
    return np.asarray(bf16_round(np.asarray(x, dtype=np.float32).astype(np.float64)),
                      dtype=np.float32).view(np.uint32).__rshift__(16).astype(np.uint16)


# --------------------------------------------------------------------- router
def route(logits: np.ndarray, k: int):
    """Top-k softmax router with renormalisation.

    ``logits`` float32 [T, E]. Returns ``ids`` int32 [T, k] (descending by
    logit, ties to the lower id) and ``weights`` float64 [T, k]:
    p = softmax(logits) over E in float64, keep the k selected, divide by
    their sum.
    """
    lg = np.asarray(logits, dtype=np.float32)
    T, E = lg.shape
    assert 1 <= k <= E
    ids = np.empty((T, k), dtype=np.int32)
    w = np.empty((T, k), dtype=np.float64)
    for t in range(T):
        order = sorted(range(E), key=lambda e: (-float(lg[t, e]), e))
        sel = order[:k]
        ids[t] = sel
        l64 = lg[t].astype(np.float64)
        p = np.exp(l64 - l64.max())
        p = p / p.sum()
        w[t] = p[sel] / p[sel].sum()
    return ids, w


# ---------------------------------------------------------------- permutation
def permute(ids: np.ndarray, E: int):
    """Stable counting sort of flat slots s = t*k + j by expert id.

    Returns dict with ``offsets`` int32 [E+1] (exclusive prefix sum of
    per-expert counts), ``sorted_slot`` int32 [S] (row r holds slot
    sorted_slot[r]; slots of one expert in ascending order),
    ``slot_to_row`` int32 [S] (inverse permutation), ``active`` int32 (experts
    with at least one row, ascending) and ``counts`` int32 [E].
    """
    flat = np.asarray(ids, dtype=np.int64).reshape(-1)
    S = flat.size
    counts = np.zeros(E, dtype=np.int64)
    for e in flat:
        counts[e] += 1
    offsets = np.zeros(E + 1, dtype=np.int64)
    for e in range(E):
        offsets[e + 1] = offsets[e] + counts[e]
    cursor = offsets[:E].copy()
    sorted_slot = np.empty(S, dtype=np.int64)
    for s in range(S):
        e = flat[s]
        sorted_slot[cursor[e]] = s
        cursor[e] += 1
    slot_to_row = np.empty(S, dtype=np.int64)
    slot_to_row[sorted_slot] = np.arange(S)
    active = np.array([e for e in range(E) if counts[e] > 0], dtype=np.int32)
    return dict(offsets=offsets.astype(np.int32), sorted_slot=sorted_slot.astype(np.int32),
                slot_to_row=slot_to_row.astype(np.int32), active=active,
                counts=counts.astype(np.int32))


# ---------------------------------------------------------------------- GEMMs
def silu(x: np.ndarray) -> np.ndarray:
    """x / (1 + exp(-x)) in float64."""
    x = np.asarray(x, dtype=np.float64)
    with np.errstate(over="ignore"):
        return x / (1.0 + np.exp(-x))


def swiglu(G: np.ndarray) -> np.ndarray:
    """[M, 2F] -> [M, F]: silu(G[:, :F]) * G[:, F:] (gate first, then up)."""
    F = G.shape[1] // 2
    return silu(G[:, :F]) * G[:, F:]


def grouped_gemm(A: np.ndarray, offsets: np.ndarray, W: list, epilogue: str = "none") -> np.ndarray:
    """Grouped GEMM on float64 operands: rows offsets[e]:offsets[e+1] of A times W[e]^T.

    ``A`` float64 [rows, K]; ``W`` a list (or callable e -> array) giving the
    float64 [N, K] matrix of expert e. Experts with no rows are skipped and
    their weights are never materialised. ``epilogue`` "swiglu" applies
    :func:`swiglu` to each expert's product.
    """
    E = len(offsets) - 1
    get = W if callable(W) else (lambda e: W[e])
    out = None
    for e in range(E):
        r0, r1 = int(offsets[e]), int(offsets[e + 1])
        if r1 == r0:
            continue
        We = get(e)
        P = A[r0:r1] @ We.T
        if epilogue == "swiglu":
            P = swiglu(P)
        if out is None:
            out = np.zeros((A.shape[0], P.shape[1]), dtype=np.float64)
        out[r0:r1] = P
    if out is None:
        n = get(0).shape[0]
        out = np.zeros((A.shape[0], n // 2 if epilogue == "swiglu" else n), dtype=np.float64)
    return out


def unpermute_reduce(Y: np.ndarray, slot_to_row: np.ndarray, w: np.ndarray) -> np.ndarray:
    """out[t] = sum_j w[t, j] * Y[slot_to_row[t*k + j]] in float64 (j ascending)."""
    T, k = w.shape
    out = np.zeros((T, Y.shape[1]), dtype=np.float64)
    for t in range(T):
        for j in range(k):
            out[t] += w[t, j] * Y[slot_to_row[t * k + j]]
    return out


# -------------------------------------------------------- activation formats
def fp8_roundtrip_bf16(x: np.ndarray) -> np.ndarray:
    """FP8 E4M3 activations dequantized to bf16 (per-tensor scale), float64 result.

    s_a = fp32(amax / 448) with amax over the finite entries (1 if that amax is 0);
    c = E4M3_RNE(min(|fp32(x / s_a)|, 448)) with the sign of x (so +-Inf saturates
    to +-448); x' = bf16(fp32(E4M3[c] * s_a)); NaN stays NaN.
    """
    x = np.asarray(x, dtype=np.float32)
    fin = np.abs(x[np.isfinite(x)])
    amax = np.float32(fin.max()) if fin.size else np.float32(0)
    s_a = np.float32(1.0) if amax == 0 else np.float32(amax / np.float32(nvfp4.E4M3_MAX))
    with np.errstate(invalid="ignore"):
        r = (x / s_a).astype(np.float32)
    mag = nvfp4.e4m3_rne(np.minimum(np.abs(np.nan_to_num(r, nan=0.0)), np.float32(nvfp4.E4M3_MAX)))
    v = np.where(np.signbit(r), -1.0, 1.0) * nvfp4.E4M3_TABLE[mag]
    prod = (v.astype(np.float32) * s_a).astype(np.float32)
    out = bf16_round(prod.astype(np.float64))
    return np.where(np.isnan(x), np.nan, out)


def quantize_rows_nvfp4(x: np.ndarray, g=None):
    """W4A4 activations: NVFP4-quantize [T, H] row-wise groups with one dynamic g."""
    return nvfp4.quantize(np.asarray(x, dtype=np.float32), g)


def round_h(h: np.ndarray, mode: str):
    """Rounding point of h between the two GEMMs. Returns (h as the down GEMM reads it,
    float64; the quantized triple or pair, or None).

    w4a16: h rounded to bf16. w4a4: h (as float32) NVFP4-quantized as one tensor with one
    dynamic global scale, like the token activations. mxfp4: h MXFP4-quantized (no
    per-tensor scale).
    """
    if mode == "w4a16":
        return bf16_round(h), None
    fmt = mxfp4 if mode == "mxfp4" else nvfp4
    hq = fmt.quantize(np.asarray(h, dtype=np.float64).astype(np.float32))
    return fmt.dequantize(*hq), hq


# ------------------------------------------------------------------ the layer
def moe_layer(x, logits, k, w13, w2, mode="w4a16", return_stages=False):
    """The whole MoE layer in float64 with the rounding points fixed above.

    ``x`` float32 [T, H] holding bf16 values (the activations as the GPU sees
    them); ``logits`` float32 [T, E]; ``w13`` / ``w2``: callables e -> (packed,
    scales, g) NVFP4 triples of W13_e [2F, H] and W2_e [H, F] (so that only
    touched experts are decoded), or (packed, scales) MXFP4 pairs in mode
    "mxfp4". ``mode`` "w4a16", "w4a4" (NVFP4 activations and h) or "mxfp4"
    (MXFP4 weights, activations and h).
    Returns the bf16-rounded output [T, H] as float64 (and the stages).
    """
    x = np.asarray(x, dtype=np.float32)
    T, H = x.shape
    E = logits.shape[1]
    ids, w = route(logits, k)
    perm = permute(ids, E)
    tok = perm["sorted_slot"].astype(np.int64) // k
    st = dict(ids=ids, w=w, perm=perm)
    assert mode in ("w4a16", "w4a4", "mxfp4"), mode
    fmt = mxfp4 if mode == "mxfp4" else nvfp4
    if mode == "w4a16":
        A = x.astype(np.float64)[tok]
    else:
        qa = quantize_rows_nvfp4(x) if mode == "w4a4" else mxfp4.quantize(x)
        st["xq"] = qa
        A = fmt.dequantize(*qa)[tok]
    dq13 = lambda e: fmt.dequantize(*w13(e))
    dq2 = lambda e: fmt.dequantize(*w2(e))
    h = grouped_gemm(A, perm["offsets"], dq13, "swiglu")
    st["h_exact"] = h
    h, hq = round_h(h, mode)
    if hq is not None:
        st["hq"] = hq
    st["h"] = h
    Y = grouped_gemm(h, perm["offsets"], dq2, "none")
    st["Y"] = Y
    out = bf16_round(unpermute_reduce(Y, perm["slot_to_row"], w))
    return (out, st) if return_stages else out
