"""The MoE layer as a sequence of C ABI calls (route -> up/gate + SwiGLU -> down -> reduce).

This module only sequences the library calls and allocates their outputs with torch; all
arithmetic runs in the HIP kernels behind include/nvfp4moe.h.
"""
from __future__ import annotations

from dataclasses import dataclass

import torch

from . import inputs, ops


@dataclass
class NVFP4Experts:
    """NVFP4 expert weights: W13_e = [2F, H] (gate rows first), W2_e = [H, F], in the pages'
    row-major storage and, for the GEMMs, in the library's tiled storage."""
    w13_packed: torch.Tensor   # uint8 [E, 2F, H/2]
    w13_scales: torch.Tensor   # uint8 [E, 2F, H/16]
    w13_g: torch.Tensor        # f32 [E]
    w2_packed: torch.Tensor    # uint8 [E, H, F/2]
    w2_scales: torch.Tensor    # uint8 [E, H, F/16]
    w2_g: torch.Tensor         # f32 [E]
    w13_t: ops.TiledWeights = None
    w2_t: ops.TiledWeights = None

    @property
    def E(self):
        return self.w13_packed.shape[0]

    def w13(self, e):
        return self.w13_packed[e], self.w13_scales[e], self.w13_g[e]

    def w2(self, e):
        return self.w2_packed[e], self.w2_scales[e], self.w2_g[e]


def quantize_experts(wl: inputs.Workload, device="cuda", experts=None) -> NVFP4Experts:
    """Generate the workload's seeded FP32 expert weights one expert at a time on ``device``
    and quantize each with the library's nvfp4_quantize twice: into the row-major storage
    (kept for users and checks) and straight into the tiled storage the GEMMs read."""
    E, H, F = wl.E, wl.H, wl.F
    experts = range(E) if experts is None else experts
    u8 = dict(dtype=torch.uint8, device=device)
    w = NVFP4Experts(
        torch.zeros((E, 2 * F, H // 2), **u8), torch.zeros((E, 2 * F, H // 16), **u8),
        torch.ones((E,), dtype=torch.float32, device=device),
        torch.zeros((E, H, F // 2), **u8), torch.zeros((E, H, F // 16), **u8),
        torch.ones((E,), dtype=torch.float32, device=device))
    lib = ops._lib.load()
    w.w13_t = ops.TiledWeights(torch.zeros((E, lib.nvfp4_tiled_codes_bytes(2 * F, H)), **u8),
                               torch.zeros((E, lib.nvfp4_tiled_scales_bytes(2 * F, H)), **u8), w.w13_g, 2 * F, H)
    w.w2_t = ops.TiledWeights(torch.zeros((E, lib.nvfp4_tiled_codes_bytes(H, F)), **u8),
                              torch.zeros((E, lib.nvfp4_tiled_scales_bytes(H, F)), **u8), w.w2_g, H, F)
    for e in experts:
        for name, rm, t, gg in (("w13", (w.w13_packed, w.w13_scales), w.w13_t, w.w13_g),
                                ("w2", (w.w2_packed, w.w2_scales), w.w2_t, w.w2_g)):
            wf = inputs.expert_weight_fp32(wl, name, e, device)
            ops.nvfp4_quantize(wf, out=(rm[0][e], rm[1][e], gg[e:e + 1]))
            ops.nvfp4_quantize(wf, out=(t.codes[e], t.scales[e], gg[e:e + 1]), tiled=True)
    return w


def moe_forward(x: torch.Tensor, logits: torch.Tensor, k: int, w: NVFP4Experts, mode: int = ops.W4A16,
                fp8_acts: bool = False, keep: bool = False, combine: bool = False):
    """One MoE layer forward. ``x`` bf16 [T, H]; ``logits`` f32 [T, E].

    Returns the bf16 output [T, H]; with ``keep`` a dict of every stage's tensors. With
    ``combine`` the down GEMM and the weighted reduce run as one call
    (moe_grouped_gemm_nvfp4_combine; same output bits, no Y in the stages).
    """
    st = {}
    T = x.shape[0]
    S = T * k
    if mode == ops.W4A16:
        # routing, permutation and the token rows' preparation (after the FP8 round trip when
        # asked): one launch for up to 16 tokens
        r = ops.moe_dispatch_w4a16(logits, x, k, fp8_act=fp8_acts)
        if keep and fp8_acts:   # the rows the GEMM sees, for inspection only
            st["x_fp8"] = ops.act_fp8_e4m3_roundtrip(x)
    else:
        if fp8_acts:
            x = ops.act_fp8_e4m3_roundtrip(x)
            st["x_fp8"] = x
        r = ops.moe_route_permute(logits, k)
    st.update(r)
    common = dict(expert_offsets=r["expert_offsets"], active_experts=r["active_experts"],
                  n_active=r["n_active"])
    if mode == ops.W4A16:
        h = ops.moe_grouped_gemm_nvfp4(ops.W4A16_PREPARED, ops.EPI_SWIGLU, r["x_prep"], w.w13_t,
                                       gather_index=r["sorted_slot"], gather_div=k, rows=S, a_rows=T,
                                       out_dtype=torch.bfloat16, **common)
        if combine:
            out = ops.moe_grouped_gemm_nvfp4_combine(ops.W4A16, h, w.w2_t, sorted_slot=r["sorted_slot"],
                                                     slot_to_row=r["slot_to_row"], topk_w=r["topk_w"], **common)
        else:
            y = ops.moe_grouped_gemm_nvfp4(ops.W4A16, ops.EPI_NONE, h, w.w2_t,
                                           rows=S, out_dtype=torch.float32, **common)
    else:
        xq, xs, xg = ops.nvfp4_quantize(x)
        st.update(xq=xq, xs=xs, xg=xg)
        h, amax = ops.moe_grouped_gemm_nvfp4(ops.W4A4, ops.EPI_SWIGLU, xq, w.w13_t,
                                             a_scales=xs, a_g=xg, gather_index=r["sorted_slot"],
                                             gather_div=k, rows=S, out_dtype=torch.float32,
                                             want_amax=True, **common)
        hq, hs, hg = ops.nvfp4_quantize(h, amax=amax)
        st.update(h_amax=amax, hq=hq, hs=hs, hg=hg)
        if combine:
            out = ops.moe_grouped_gemm_nvfp4_combine(ops.W4A4, hq, w.w2_t, sorted_slot=r["sorted_slot"],
                                                     slot_to_row=r["slot_to_row"], topk_w=r["topk_w"],
                                                     a_scales=hs, a_g=hg, **common)
        else:
            y = ops.moe_grouped_gemm_nvfp4(ops.W4A4, ops.EPI_NONE, hq, w.w2_t,
                                           a_scales=hs, a_g=hg, rows=S, out_dtype=torch.float32, **common)
    if not combine:
        out = ops.moe_unpermute_reduce(y, r["slot_to_row"], r["topk_w"])
    if keep:
        st.update(h=h, out=out, **({} if combine else dict(y=y)))
        return out, st
    return out


@dataclass
class MXFP4Experts:
    """MXFP4 expert weights (group-32 UE8M0 scales, no per-tensor scale), same shapes as
    NVFP4Experts: row-major as quantized, and tiled for the GEMM."""
    w13_packed: torch.Tensor   # uint8 [E, 2F, H/2]
    w13_scales: torch.Tensor   # uint8 [E, 2F, H/32]
    w2_packed: torch.Tensor    # uint8 [E, H, F/2]
    w2_scales: torch.Tensor    # uint8 [E, H, F/32]
    w13_t: ops.MxTiledWeights = None
    w2_t: ops.MxTiledWeights = None

    @property
    def E(self):
        return self.w13_packed.shape[0]


def quantize_experts_mxfp4(wl: inputs.Workload, device="cuda") -> MXFP4Experts:
    """The workload's seeded FP32 expert weights (the same values quantize_experts starts
    from), quantized one expert at a time with mxfp4_quantize, then tiled."""
    E, H, F = wl.E, wl.H, wl.F
    u8 = dict(dtype=torch.uint8, device=device)
    w = MXFP4Experts(torch.empty((E, 2 * F, H // 2), **u8), torch.empty((E, 2 * F, H // 32), **u8),
                     torch.empty((E, H, F // 2), **u8), torch.empty((E, H, F // 32), **u8))
    for e in range(E):
        p, sc = ops.mxfp4_quantize(inputs.expert_weight_fp32(wl, "w13", e, device))
        w.w13_packed[e].copy_(p)
        w.w13_scales[e].copy_(sc)
        p, sc = ops.mxfp4_quantize(inputs.expert_weight_fp32(wl, "w2", e, device))
        w.w2_packed[e].copy_(p)
        w.w2_scales[e].copy_(sc)
    w.w13_t = ops.mxfp4_weights_tile(w.w13_packed, w.w13_scales)
    w.w2_t = ops.mxfp4_weights_tile(w.w2_packed, w.w2_scales)
    return w


def moe_forward_mxfp4(x: torch.Tensor, logits: torch.Tensor, k: int, w: MXFP4Experts,
                      keep: bool = False, combine: bool = False):
    """One MoE layer forward in MXFP4 W4A4: token rows and h are MXFP4-quantized (one UE8M0
    scale per 32 elements, no per-tensor scale, so the up/gate GEMM's epilogue writes h as
    MXFP4 directly); both GEMMs run on the scaled FP4 matrix cores. ``x`` bf16 [T, H];
    ``logits`` f32 [T, E]."""
    st = {}
    r = ops.moe_route_permute(logits, k)
    st.update(r)
    S = x.shape[0] * k
    common = dict(expert_offsets=r["expert_offsets"], active_experts=r["active_experts"],
                  n_active=r["n_active"])
    xq, xs = ops.mxfp4_quantize(x)
    hq, hs = ops.moe_grouped_gemm_mxfp4_swiglu_q(xq, xs, w.w13_t, gather_index=r["sorted_slot"],
                                                 gather_div=k, rows=S, **common)
    if combine:
        out = ops.moe_grouped_gemm_mxfp4_combine(hq, hs, w.w2_t, sorted_slot=r["sorted_slot"],
                                                 slot_to_row=r["slot_to_row"], topk_w=r["topk_w"], **common)
    else:
        y = ops.moe_grouped_gemm_mxfp4(ops.EPI_NONE, hq, hs, w.w2_t, rows=S, out_dtype=torch.float32, **common)
        out = ops.moe_unpermute_reduce(y, r["slot_to_row"], r["topk_w"])
    if keep:
        st.update(xq=xq, xs=xs, hq=hq, hs=hs, out=out, **({} if combine else dict(y=y)))
        return out, st
    return out
