"""Thin PyTorch binding of libnvfp4moe: one function per C ABI call, same names.

Only argument marshalling happens here: tensors are checked for device/dtype/shape,
outputs and workspaces are allocated with torch (device memory and streams are all torch
is used for), and the C call is made on the current HIP stream. Every step of the
computation runs in the library's HIP kernels; a failed call raises NVFP4MoEError.
"""
from __future__ import annotations

import ctypes
import math
from dataclasses import dataclass

import torch

from . import _lib
from ._lib import (BF16, EPI_NONE, EPI_SWIGLU, F32, PATH_MFMA, PATH_NONE, PATH_STREAM,  # noqa: F401
                   W4A4, W4A16, W4A16_PREPARED)


def _ptr(t):
    return ctypes.c_void_p(t.data_ptr()) if t is not None else None


def _stream():
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _dev(*ts):
    for t in ts:
        if t is not None and not t.is_cuda:
            raise ValueError("all tensors must be on the GPU")


def _ws(nbytes, device):
    return torch.empty(max(int(nbytes), 1), dtype=torch.uint8, device=device)


_DT = {torch.float32: F32, torch.bfloat16: BF16}


def nvfp4_quantize(x: torch.Tensor, g: torch.Tensor | None = None, amax: torch.Tensor | None = None,
                   out: tuple | None = None, tiled: bool = False):
    """Quantize [R, C] or [B, R, C] float32/bf16 to NVFP4.

    Row-major (default) -> (packed [B, R, C/2], scales [B, R, C/16], g [B]) (the batch dim
    dropped for a 2-D x); ``tiled`` -> a TiledWeights in the storage moe_grouped_gemm_nvfp4
    reads, written by the same call (R % 16 == 0).
    ``g``: optional device float[B] global scales; ``amax``: optional device float[B]
    finite max |x| per matrix (used when ``g`` is None); ``out``: optional preallocated
    (packed, scales, g) to write into (contiguous; row-major shapes, or the tiled byte counts).
    """
    _dev(x, g, amax)
    squeeze = x.dim() == 2
    x3 = x.unsqueeze(0) if squeeze else x
    x3 = x3.contiguous()
    B, R, C = x3.shape
    lib = _lib.load()
    if tiled:
        ncb, nsb = lib.nvfp4_tiled_codes_bytes(R, C), lib.nvfp4_tiled_scales_bytes(R, C)
        shapes = ((B, ncb), (B, nsb))
    else:
        shapes = ((B, R, C // 2), (B, R, C // 16))
    if out is not None:
        packed, scales, g_out = out
        assert packed.is_contiguous() and scales.is_contiguous() and g_out.is_contiguous()
        assert packed.numel() == math.prod(shapes[0]) and scales.numel() == math.prod(shapes[1])
        assert g_out.numel() == B
    else:
        packed = torch.empty(shapes[0], dtype=torch.uint8, device=x.device)
        scales = torch.empty(shapes[1], dtype=torch.uint8, device=x.device)
        g_out = torch.empty((B,), dtype=torch.float32, device=x.device)
    ws = _ws(lib.nvfp4_quantize_workspace_size(B, R, C), x.device)
    layout = _lib.LAYOUT_TILED if tiled else _lib.LAYOUT_ROW_MAJOR
    st = lib.nvfp4_quantize(_ptr(x3), _DT[x3.dtype], B, R, C, _ptr(g), _ptr(amax), layout, _ptr(packed),
                            _ptr(scales), _ptr(g_out), _ptr(ws), ws.numel(), _stream())
    _lib.check("nvfp4_quantize", st)
    if tiled:
        return TiledWeights(packed, scales, g_out, R, C)
    if squeeze and out is None:
        return packed[0], scales[0], g_out
    return packed, scales, g_out


@dataclass
class TiledWeights:
    """B NVFP4 matrices [R, C] in the tiled storage of nvfp4_weights_tile, with their
    per-matrix global scales: what moe_grouped_gemm_nvfp4 takes as expert weights."""
    codes: torch.Tensor    # uint8 [B, nvfp4_tiled_codes_bytes(R, C)]
    scales: torch.Tensor   # uint8 [B, nvfp4_tiled_scales_bytes(R, C)]
    g: torch.Tensor        # float32 [B]
    R: int
    C: int

    @property
    def B(self):
        return self.codes.shape[0]


def nvfp4_weights_tile(packed: torch.Tensor, scales: torch.Tensor, g: torch.Tensor) -> TiledWeights:
    """Reorder NVFP4 weights packed [B, R, C/2] + scales [B, R, C/16] (or one [R, ...]
    matrix) into the tiled storage the grouped GEMM reads; a byte permutation with zero
    padding (include/nvfp4moe.h). ``g`` float32 [B] is carried along unchanged."""
    _dev(packed, scales, g)
    p3 = (packed.unsqueeze(0) if packed.dim() == 2 else packed).contiguous()
    s3 = (scales.unsqueeze(0) if scales.dim() == 2 else scales).contiguous()
    B, R, Ch = p3.shape
    C = 2 * Ch
    assert s3.shape == (B, R, C // 16), (s3.shape, p3.shape)
    lib = _lib.load()
    cb, sb = lib.nvfp4_tiled_codes_bytes(R, C), lib.nvfp4_tiled_scales_bytes(R, C)
    if cb == 0 or sb == 0:
        raise _lib.NVFP4MoEError("nvfp4_weights_tile", _lib.ERR_INVALID_ARG, f"unsupported shape R={R} C={C}")
    codes = torch.empty((B, cb), dtype=torch.uint8, device=packed.device)
    sc = torch.empty((B, sb), dtype=torch.uint8, device=packed.device)
    st = lib.nvfp4_weights_tile(_ptr(p3), _ptr(s3), B, R, C, _ptr(codes), _ptr(sc), _stream())
    _lib.check("nvfp4_weights_tile", st)
    g = g.reshape(-1).float().contiguous()
    assert g.numel() == B
    return TiledWeights(codes, sc, g, R, C)


def moe_route_permute(logits: torch.Tensor, k: int):
    """Router + permutation. Returns a dict of device tensors (see include/nvfp4moe.h)."""
    _dev(logits)
    logits = logits.contiguous().float()
    T, E = logits.shape
    dev = logits.device
    i32 = dict(dtype=torch.int32, device=dev)
    out = dict(
        topk_ids=torch.empty((T, k), **i32),
        topk_w=torch.empty((T, k), dtype=torch.float32, device=dev),
        expert_offsets=torch.empty((E + 1,), **i32),
        sorted_slot=torch.empty((T * k,), **i32),
        slot_to_row=torch.empty((T * k,), **i32),
        active_experts=torch.empty((E,), **i32),
        n_active=torch.empty((1,), **i32),
    )
    lib = _lib.load()
    ws = _ws(lib.moe_route_permute_workspace_size(T, E, k), dev)
    st = lib.moe_route_permute(_ptr(logits), T, E, k, _ptr(out["topk_ids"]), _ptr(out["topk_w"]),
                               _ptr(out["expert_offsets"]), _ptr(out["sorted_slot"]),
                               _ptr(out["slot_to_row"]), _ptr(out["active_experts"]),
                               _ptr(out["n_active"]), _ptr(ws), ws.numel(), _stream())
    _lib.check("moe_route_permute", st)
    return out


def moe_grouped_gemm_nvfp4(mode: int, epi: int, a: torch.Tensor, w: TiledWeights,
                           expert_offsets: torch.Tensor, active_experts: torch.Tensor,
                           n_active: torch.Tensor, *,
                           a_scales: torch.Tensor | None = None, a_g: torch.Tensor | None = None,
                           gather_index: torch.Tensor | None = None, gather_div: int = 1,
                           rows: int | None = None, out_dtype=torch.bfloat16,
                           want_amax: bool = False, out: torch.Tensor | None = None,
                           a_rows: int | None = None):
    """Grouped NVFP4 GEMM (+ SwiGLU). ``w``: E expert matrices [Nw, K] (tiled); ``a`` bf16
    [a_rows, K] (W4A16), packed uint8 [a_rows, K/2] (W4A4), or the ``x_prep`` bytes of
    moe_dispatch_w4a16 (W4A16_PREPARED, with ``a_rows`` = its T). Returns out (and amax)."""
    _dev(a, w.codes, w.scales, w.g, expert_offsets, active_experts, n_active, a_scales, a_g, gather_index)
    E, Nw, K = w.B, w.R, w.C
    if a_rows is None:
        if mode == W4A16_PREPARED:
            raise ValueError("W4A16_PREPARED needs a_rows (the T of moe_dispatch_w4a16)")
        a_rows = a.shape[0]
    if rows is None:
        rows = gather_index.numel() if gather_index is not None else a_rows
    ncol = Nw // 2 if epi == EPI_SWIGLU else Nw
    if out is None:
        out = torch.empty((rows, ncol), dtype=out_dtype, device=a.device)
    amax = torch.empty((1,), dtype=torch.float32, device=a.device) if want_amax else None
    lib = _lib.load()
    ws = _ws(lib.moe_grouped_gemm_workspace_size(mode, a_rows, rows, E, Nw, K), a.device)
    st = lib.moe_grouped_gemm_nvfp4(
        mode, epi, _ptr(a), _ptr(a_scales), _ptr(a_g), a_rows, _ptr(gather_index), int(gather_div),
        _ptr(w.codes), _ptr(w.scales), _ptr(w.g), _ptr(expert_offsets), _ptr(active_experts),
        _ptr(n_active), E, rows, Nw, K, _ptr(out), _DT[out.dtype], _ptr(amax), _ptr(ws), ws.numel(),
        _stream())
    _lib.check("moe_grouped_gemm_nvfp4", st)
    return (out, amax) if want_amax else out


def moe_dispatch_w4a16(logits: torch.Tensor, x: torch.Tensor, k: int, fp8_act: bool = False):
    """moe_route_permute of ``logits`` [T, E] plus the W4A16 preparation of the token rows
    ``x`` [T, H] bf16 (after the FP8 E4M3 round trip with ``fp8_act``). Returns the routing
    dict of moe_route_permute with ``x_prep``: the bytes moe_grouped_gemm_nvfp4 reads in mode
    W4A16_PREPARED (a_rows = T, K = H)."""
    _dev(logits, x)
    logits = logits.contiguous().float()
    x = x.contiguous()
    T, E = logits.shape
    H = x.shape[1]
    dev = logits.device
    i32 = dict(dtype=torch.int32, device=dev)
    out = dict(
        topk_ids=torch.empty((T, k), **i32),
        topk_w=torch.empty((T, k), dtype=torch.float32, device=dev),
        expert_offsets=torch.empty((E + 1,), **i32),
        sorted_slot=torch.empty((T * k,), **i32),
        slot_to_row=torch.empty((T * k,), **i32),
        active_experts=torch.empty((E,), **i32),
        n_active=torch.empty((1,), **i32),
    )
    lib = _lib.load()
    out["x_prep"] = torch.empty((lib.moe_prepared_act_bytes(T, H),), dtype=torch.uint8, device=dev)
    ws = _ws(lib.moe_dispatch_w4a16_workspace_size(T, E, k, H, int(fp8_act)), dev)
    st = lib.moe_dispatch_w4a16(_ptr(logits), _ptr(x), T, E, k, H, int(fp8_act), _ptr(out["topk_ids"]),
                                _ptr(out["topk_w"]), _ptr(out["expert_offsets"]), _ptr(out["sorted_slot"]),
                                _ptr(out["slot_to_row"]), _ptr(out["active_experts"]), _ptr(out["n_active"]),
                                _ptr(out["x_prep"]), _ptr(ws), ws.numel(), _stream())
    _lib.check("moe_dispatch_w4a16", st)
    return out


def moe_grouped_gemm_nvfp4_combine(mode: int, a: torch.Tensor, w: TiledWeights, expert_offsets: torch.Tensor,
                                   active_experts: torch.Tensor, n_active: torch.Tensor, sorted_slot: torch.Tensor,
                                   slot_to_row: torch.Tensor, topk_w: torch.Tensor, *,
                                   a_scales: torch.Tensor | None = None, a_g: torch.Tensor | None = None,
                                   out: torch.Tensor | None = None):
    """Down GEMM + weighted unpermute-reduce in one call: ``a`` [T*k, K] (bf16, or NVFP4
    packed for W4A4) in permuted row order, ``w`` E matrices [H, K] (tiled), routing of
    ``topk_w`` [T, k] tokens -> bf16 out [T, H]."""
    _dev(a, w.codes, w.scales, w.g, expert_offsets, active_experts, n_active, sorted_slot, slot_to_row, topk_w,
         a_scales, a_g)
    E, Nw, K = w.B, w.R, w.C
    T, k = topk_w.shape
    if out is None:
        out = torch.empty((T, Nw), dtype=torch.bfloat16, device=a.device)
    lib = _lib.load()
    ws = _ws(lib.moe_grouped_gemm_nvfp4_combine_workspace_size(mode, T, k, E, Nw, K), a.device)
    st = lib.moe_grouped_gemm_nvfp4_combine(
        mode, _ptr(a), _ptr(a_scales), _ptr(a_g), _ptr(w.codes), _ptr(w.scales), _ptr(w.g), _ptr(expert_offsets),
        _ptr(active_experts), _ptr(n_active), _ptr(sorted_slot), _ptr(slot_to_row), _ptr(topk_w.contiguous()),
        E, T, k, Nw, K, _ptr(out), _ptr(ws), ws.numel(), _stream())
    _lib.check("moe_grouped_gemm_nvfp4_combine", st)
    return out


def moe_unpermute_reduce(y: torch.Tensor, slot_to_row: torch.Tensor, topk_w: torch.Tensor,
                         out: torch.Tensor | None = None):
    """out[t] = bf16(sum_j topk_w[t, j] * y[slot_to_row[t*k + j]])."""
    _dev(y, slot_to_row, topk_w)
    T, k = topk_w.shape
    H = y.shape[1]
    if out is None:
        out = torch.empty((T, H), dtype=torch.bfloat16, device=y.device)
    lib = _lib.load()
    st = lib.moe_unpermute_reduce(_ptr(y), _DT[y.dtype], _ptr(slot_to_row), _ptr(topk_w), T, k, H,
                                  _ptr(out), _stream())
    _lib.check("moe_unpermute_reduce", st)
    return out


def act_fp8_e4m3_roundtrip(x: torch.Tensor, out: torch.Tensor | None = None):
    """FP8 E4M3 (per-tensor scale) round trip of bf16 activations, returned as bf16."""
    _dev(x)
    x = x.contiguous()
    if out is None:
        out = torch.empty_like(x)
    lib = _lib.load()
    n = x.numel()
    ws = _ws(lib.act_fp8_e4m3_roundtrip_workspace_size(n), x.device)
    st = lib.act_fp8_e4m3_roundtrip(_ptr(x), n, _ptr(out), _ptr(ws), ws.numel(), _stream())
    _lib.check("act_fp8_e4m3_roundtrip", st)
    return out


# ------------------------------------------------------------------ MXFP4 variant
def mxfp4_quantize(x: torch.Tensor):
    """Float rows [..., C] (C % 32 == 0) -> MXFP4 (packed uint8 [..., C/2], UE8M0 scales
    uint8 [..., C/32]); one scale per 32 elements, no per-tensor scale."""
    _dev(x)
    x = x.contiguous()
    C = x.shape[-1]
    R = x.numel() // C
    packed = torch.empty(x.shape[:-1] + (C // 2,), dtype=torch.uint8, device=x.device)
    scales = torch.empty(x.shape[:-1] + (C // 32,), dtype=torch.uint8, device=x.device)
    lib = _lib.load()
    st = lib.mxfp4_quantize(_ptr(x), _DT[x.dtype], R, C, _ptr(packed), _ptr(scales), _stream())
    _lib.check("mxfp4_quantize", st)
    return packed, scales


@dataclass
class MxTiledWeights:
    """B MXFP4 matrices [R, C] in the tiled storage moe_grouped_gemm_mxfp4 reads."""
    codes: torch.Tensor    # uint8 [B, nvfp4_tiled_codes_bytes(R, C)]
    scales: torch.Tensor   # uint8 [B, mxfp4_tiled_scales_bytes(R, C)]
    R: int
    C: int

    @property
    def B(self) -> int:
        return self.codes.shape[0]


def mxfp4_weights_tile(packed: torch.Tensor, scales: torch.Tensor) -> MxTiledWeights:
    """Reorder MXFP4 weights packed [B, R, C/2] + scales [B, R, C/32] (or one matrix) into
    the tiled storage; a byte permutation with zero padding (include/nvfp4moe.h)."""
    _dev(packed, scales)
    p3 = (packed.unsqueeze(0) if packed.dim() == 2 else packed).contiguous()
    s3 = (scales.unsqueeze(0) if scales.dim() == 2 else scales).contiguous()
    B, R, Ch = p3.shape
    C = 2 * Ch
    assert s3.shape == (B, R, C // 32), (s3.shape, p3.shape)
    lib = _lib.load()
    cb, sb = lib.nvfp4_tiled_codes_bytes(R, C), lib.mxfp4_tiled_scales_bytes(R, C)
    if cb == 0 or sb == 0:
        raise _lib.NVFP4MoEError("mxfp4_weights_tile", _lib.ERR_INVALID_ARG, f"unsupported shape R={R} C={C}")
    codes = torch.empty((B, cb), dtype=torch.uint8, device=packed.device)
    sc = torch.empty((B, sb), dtype=torch.uint8, device=packed.device)
    st = lib.mxfp4_weights_tile(_ptr(p3), _ptr(s3), B, R, C, _ptr(codes), _ptr(sc), _stream())
    _lib.check("mxfp4_weights_tile", st)
    return MxTiledWeights(codes, sc, R, C)


def moe_grouped_gemm_mxfp4(epi: int, a: torch.Tensor, a_scales: torch.Tensor, w: MxTiledWeights,
                           expert_offsets: torch.Tensor, active_experts: torch.Tensor,
                           n_active: torch.Tensor, *, gather_index: torch.Tensor | None = None,
                           gather_div: int = 1, rows: int | None = None, out_dtype=torch.bfloat16,
                           want_amax: bool = False, out: torch.Tensor | None = None):
    """W4A4 grouped GEMM with MXFP4 weights ``w`` (E matrices [Nw, K], tiled) and MXFP4
    activations ``a`` [a_rows, K/2] + ``a_scales`` [a_rows, K/32] (+ SwiGLU)."""
    _dev(a, a_scales, w.codes, w.scales, expert_offsets, active_experts, n_active, gather_index)
    E, Nw, K = w.B, w.R, w.C
    a_rows = a.shape[0]
    if rows is None:
        rows = gather_index.numel() if gather_index is not None else a_rows
    ncol = Nw // 2 if epi == EPI_SWIGLU else Nw
    if out is None:
        out = torch.empty((rows, ncol), dtype=out_dtype, device=a.device)
    amax = torch.empty((1,), dtype=torch.float32, device=a.device) if want_amax else None
    lib = _lib.load()
    ws = _ws(lib.moe_grouped_gemm_mxfp4_workspace_size(rows, E, Nw, K), a.device)
    st = lib.moe_grouped_gemm_mxfp4(
        epi, _ptr(a), _ptr(a_scales), a_rows, _ptr(gather_index), int(gather_div), _ptr(w.codes),
        _ptr(w.scales), _ptr(expert_offsets), _ptr(active_experts), _ptr(n_active), E, rows, Nw, K,
        _ptr(out), _DT[out.dtype], _ptr(amax), _ptr(ws), ws.numel(), _stream())
    _lib.check("moe_grouped_gemm_mxfp4", st)
    return (out, amax) if want_amax else out


def moe_grouped_gemm_mxfp4_combine(a: torch.Tensor, a_scales: torch.Tensor, w: MxTiledWeights,
                                   expert_offsets: torch.Tensor, active_experts: torch.Tensor, n_active: torch.Tensor,
                                   sorted_slot: torch.Tensor, slot_to_row: torch.Tensor, topk_w: torch.Tensor, *,
                                   out: torch.Tensor | None = None):
    """MXFP4 down GEMM + weighted unpermute-reduce in one call -> bf16 out [T, H]."""
    _dev(a, a_scales, w.codes, w.scales, expert_offsets, active_experts, n_active, sorted_slot, slot_to_row, topk_w)
    E, Nw, K = w.B, w.R, w.C
    T, k = topk_w.shape
    if out is None:
        out = torch.empty((T, Nw), dtype=torch.bfloat16, device=a.device)
    lib = _lib.load()
    ws = _ws(lib.moe_grouped_gemm_mxfp4_combine_workspace_size(T, k, E, Nw, K), a.device)
    st = lib.moe_grouped_gemm_mxfp4_combine(
        _ptr(a), _ptr(a_scales), _ptr(w.codes), _ptr(w.scales), _ptr(expert_offsets), _ptr(active_experts),
        _ptr(n_active), _ptr(sorted_slot), _ptr(slot_to_row), _ptr(topk_w.contiguous()), E, T, k, Nw, K, _ptr(out),
        _ptr(ws), ws.numel(), _stream())
    _lib.check("moe_grouped_gemm_mxfp4_combine", st)
    return out


def moe_grouped_gemm_mxfp4_swiglu_q(a: torch.Tensor, a_scales: torch.Tensor, w: MxTiledWeights,
                                    expert_offsets: torch.Tensor, active_experts: torch.Tensor,
                                    n_active: torch.Tensor, *, gather_index: torch.Tensor | None = None,
                                    gather_div: int = 1, rows: int | None = None):
    """MXFP4 up/gate GEMM + SwiGLU with h written as MXFP4 by the epilogue: returns
    (h_packed uint8 [rows, Nw/4], h_scales uint8 [rows, Nw/64])."""
    _dev(a, a_scales, w.codes, w.scales, expert_offsets, active_experts, n_active, gather_index)
    E, Nw, K = w.B, w.R, w.C
    a_rows = a.shape[0]
    if rows is None:
        rows = gather_index.numel() if gather_index is not None else a_rows
    F = Nw // 2
    hp = torch.empty((rows, F // 2), dtype=torch.uint8, device=a.device)
    hs = torch.empty((rows, F // 32), dtype=torch.uint8, device=a.device)
    lib = _lib.load()
    ws = _ws(lib.moe_grouped_gemm_mxfp4_workspace_size(rows, E, Nw, K), a.device)
    st = lib.moe_grouped_gemm_mxfp4_swiglu_q(
        _ptr(a), _ptr(a_scales), a_rows, _ptr(gather_index), int(gather_div), _ptr(w.codes), _ptr(w.scales),
        _ptr(expert_offsets), _ptr(active_experts), _ptr(n_active), E, rows, Nw, K, _ptr(hp), _ptr(hs),
        _ptr(ws), ws.numel(), _stream())
    _lib.check("moe_grouped_gemm_mxfp4_swiglu_q", st)
    return hp, hs


def mxfp8_quantize(x: torch.Tensor):
    """Float rows [..., C] (C % 32 == 0) -> MXFP8 (E4M3 codes uint8 [..., C], UE8M0 scales
    uint8 [..., C/32]); one scale per 32 elements, no per-tensor scale."""
    _dev(x)
    x = x.contiguous()
    C = x.shape[-1]
    R = x.numel() // C
    codes = torch.empty(x.shape, dtype=torch.uint8, device=x.device)
    scales = torch.empty(x.shape[:-1] + (C // 32,), dtype=torch.uint8, device=x.device)
    st = _lib.load().mxfp8_quantize(_ptr(x), _DT[x.dtype], R, C, _ptr(codes), _ptr(scales), _stream())
    _lib.check("mxfp8_quantize", st)
    return codes, scales


def mxfp8_weights_tile(codes: torch.Tensor, scales: torch.Tensor) -> MxTiledWeights:
    """Reorder MXFP8 weights codes [B, R, C] + scales [B, R, C/32] (or one matrix) into the
    tiled storage moe_grouped_gemm_mxfp8 reads (include/nvfp4moe.h)."""
    _dev(codes, scales)
    c3 = (codes.unsqueeze(0) if codes.dim() == 2 else codes).contiguous()
    s3 = (scales.unsqueeze(0) if scales.dim() == 2 else scales).contiguous()
    B, R, C = c3.shape
    assert s3.shape == (B, R, C // 32), (s3.shape, c3.shape)
    lib = _lib.load()
    cb, sb = lib.mxfp8_tiled_codes_bytes(R, C), lib.mxfp4_tiled_scales_bytes(R, C)
    if cb == 0 or sb == 0:
        raise _lib.NVFP4MoEError("mxfp8_weights_tile", _lib.ERR_INVALID_ARG, f"unsupported shape R={R} C={C}")
    tc = torch.empty((B, cb), dtype=torch.uint8, device=codes.device)
    ts = torch.empty((B, sb), dtype=torch.uint8, device=codes.device)
    st = lib.mxfp8_weights_tile(_ptr(c3), _ptr(s3), B, R, C, _ptr(tc), _ptr(ts), _stream())
    _lib.check("mxfp8_weights_tile", st)
    return MxTiledWeights(tc, ts, R, C)


def moe_grouped_gemm_mxfp8(epi: int, a: torch.Tensor, a_scales: torch.Tensor, w: MxTiledWeights,
                           expert_offsets: torch.Tensor, active_experts: torch.Tensor,
                           n_active: torch.Tensor, *, gather_index: torch.Tensor | None = None,
                           gather_div: int = 1, rows: int | None = None, out_dtype=torch.bfloat16,
                           want_amax: bool = False, out: torch.Tensor | None = None):
    """W8A8 grouped GEMM with MXFP8 weights ``w`` (E matrices [Nw, K], tiled) and MXFP8
    activations ``a`` [a_rows, K] + ``a_scales`` [a_rows, K/32] (+ SwiGLU)."""
    _dev(a, a_scales, w.codes, w.scales, expert_offsets, active_experts, n_active, gather_index)
    E, Nw, K = w.B, w.R, w.C
    a_rows = a.shape[0]
    if rows is None:
        rows = gather_index.numel() if gather_index is not None else a_rows
    ncol = Nw // 2 if epi == EPI_SWIGLU else Nw
    if out is None:
        out = torch.empty((rows, ncol), dtype=out_dtype, device=a.device)
    amax = torch.empty((1,), dtype=torch.float32, device=a.device) if want_amax else None
    lib = _lib.load()
    ws = _ws(lib.moe_grouped_gemm_mxfp8_workspace_size(rows, E, Nw, K), a.device)
    st = lib.moe_grouped_gemm_mxfp8(
        epi, _ptr(a), _ptr(a_scales), a_rows, _ptr(gather_index), int(gather_div), _ptr(w.codes),
        _ptr(w.scales), _ptr(expert_offsets), _ptr(active_experts), _ptr(n_active), E, rows, Nw, K,
        _ptr(out), _DT[out.dtype], _ptr(amax), _ptr(ws), ws.numel(), _stream())
    _lib.check("moe_grouped_gemm_mxfp8", st)
    return (out, amax) if want_amax else out


def last_dispatch() -> int:
    return _lib.load().nvfp4moe_last_dispatch()
