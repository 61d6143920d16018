"""Plant plausible mistakes in the oracle (CPU only) and check that a pin catches each.

Every case monkeypatches one oracle function with a subtly wrong version (a
swapped nibble order, a dropped global scale, a transposed or wrong operand,
the wrong tie rule, an unstable sort, a wrong MX exponent bias or rule...) and
runs the pin that should expose it; the pin must fail.
"""
import numpy as np
import pytest

import oracle.moe as moe
import oracle.mxfp4 as mxfp4
import oracle.mxfp8 as mxfp8
import oracle.nvfp4 as nvfp4
import tests.test_oracle_moe as tm
import tests.test_oracle_mxfp4 as tx
import tests.test_oracle_mxfp8 as t8
import tests.test_oracle_nvfp4 as tn


def _high_nibble_first(packed):
    p = np.asarray(packed, dtype=np.uint8)
    out = np.empty(p.shape[:-1] + (p.shape[-1] * 2,), dtype=np.uint8)
    out[..., 0::2] = p >> 4
    out[..., 1::2] = p & 0x0F
    return out


def _rne_ties_up(x, grid):
    x = np.asarray(x, dtype=np.float64)
    hi = np.clip(np.searchsorted(grid, x, side="left"), 0, len(grid) - 1)
    lo = np.clip(hi - 1, 0, len(grid) - 1)
    mid = (grid[lo] + grid[hi]) * 0.5
    out = np.where(x < mid, lo, hi)
    return np.where(x >= grid[-1], len(grid) - 1, out).astype(np.uint8)


def _route_ties_high(logits, k):
    lg = np.asarray(logits, dtype=np.float32)
    ids, w = moe.__dict__["_orig_route"](lg, k)
    T, E = lg.shape
    for t in range(T):
        order = sorted(range(E), key=lambda e: (-float(lg[t, e]), -e))
        ids[t] = order[:k]
    return ids, w


def _unstable_permute(ids, E):
    p = moe.__dict__["_orig_permute"](ids, E)
    ss = p["sorted_slot"].copy()
    for e in range(E):
        a, b = p["offsets"][e], p["offsets"][e + 1]
        ss[a:b] = ss[a:b][::-1]
    p["sorted_slot"] = ss
    p["slot_to_row"] = np.argsort(ss).astype(np.int32)
    return p


def _gemm_wrong_expert(A, offsets, W, epilogue="none"):
    get = W if callable(W) else (lambda e: W[e])
    E = len(offsets) - 1
    return moe.__dict__["_orig_grouped_gemm"](A, offsets, lambda e: get((e + 1) % E), epilogue)


def _div_by_reciprocal(a, b):
    with np.errstate(divide="ignore", invalid="ignore", over="ignore"):
        r = (np.float32(1) / np.asarray(b, dtype=np.float32)).astype(np.float32)
        return (np.asarray(a, dtype=np.float32) * r).astype(np.float32)


def _h_not_requantized(h, mode):
    if mode == "w4a4":
        return moe.bf16_round(h), None
    return moe.__dict__["_orig_round_h"](h, mode)


def _quantize_rows_own_g(x, g=None):
    """Each row NVFP4-quantized with its own dynamic global scale; returns the codes, the
    scales and the per-row scales."""
    x = np.asarray(x, dtype=np.float32)
    parts = [nvfp4.quantize(x[r:r + 1]) for r in range(x.shape[0])]
    return (np.concatenate([p[0] for p in parts]), np.concatenate([p[1] for p in parts]),
            np.array([p[2] for p in parts], dtype=np.float32))


def _h_per_row_g(h, mode):
    if mode == "w4a4":
        p, s, g = _quantize_rows_own_g(np.asarray(h, dtype=np.float64).astype(np.float32))
        return nvfp4.dequantize(p, s, 1.0) * g.astype(np.float64)[:, None], (p, s, g[0])
    return moe.__dict__["_orig_round_h"](h, mode)


def _x_per_row_g(x, g=None):
    p, s, gr = _quantize_rows_own_g(x)
    return p, s, gr[0]


MUTATIONS = [
    ("quantize divides by a reciprocal", nvfp4, "div_f32", _div_by_reciprocal,
     lambda: tn.test_quantize_exact_midpoints_divide_correctly(3 * 2.0 ** -10)),
    ("w4a4 layer skips h re-quantization", moe, "round_h", _h_not_requantized,
     tm.test_layer_w4a4_with_one_expert_is_a_dense_nvfp4_ffn),
    ("w4a4 layer quantizes h with a per-row g", moe, "round_h", _h_per_row_g,
     tm.test_layer_w4a4_with_one_expert_is_a_dense_nvfp4_ffn),
    ("w4a4 layer quantizes x with a per-row g", moe, "quantize_rows_nvfp4", _x_per_row_g,
     tm.test_layer_w4a4_with_one_expert_is_a_dense_nvfp4_ffn),
    ("unpack high nibble first", nvfp4, "unpack_fp4", _high_nibble_first, tn.test_pack_low_nibble_first),
    ("e2m1 table 1.5<->2 swapped", nvfp4, "E2M1_TABLE",
     nvfp4.E2M1_TABLE[[0, 1, 2, 4, 3, 5, 6, 7, 8, 9, 10, 12, 11, 13, 14, 15]],
     tn.test_e2m1_table_matches_ocp_value_set),
    ("dequantize drops g", nvfp4, "dequantize",
     lambda p, s, g: nvfp4.__dict__["_orig_dequantize"](p, s, np.float32(1)), tn.test_dequantize_hand_example),
    ("e4m3 ties away from zero", nvfp4, "e4m3_rne",
     lambda r: _rne_ties_up(r, nvfp4._E4M3_POS), tn.test_e4m3_rne_matches_torch_cast),
    ("e2m1 ties away from zero", nvfp4, "e2m1_rne_sat",
     lambda x: _rne_ties_up(np.abs(np.asarray(x, np.float64)), nvfp4._E2M1_POS),
     tn.test_e2m1_rne_ties_and_saturation),
    ("global scale without the 6*448", nvfp4, "GLOBAL_DENOM", np.float32(448),
     tn.test_quantize_grid_inputs_roundtrip_exactly_dynamic_g),
    ("router ties to the higher id", moe, "route", _route_ties_high,
     lambda: tm.test_route_against_iterated_argmax_and_torch_softmax(16, 8, 2)),
    ("unstable permutation", moe, "permute", _unstable_permute,
     lambda: tm.test_permute_matches_stable_argsort(300, 4, 3)),
    ("grouped gemm uses the next expert", moe, "grouped_gemm", _gemm_wrong_expert,
     tm.test_grouped_gemm_exact_rationals_tiny),
    ("swiglu with up first", moe, "swiglu",
     lambda G: moe.silu(G[:, G.shape[1] // 2:]) * G[:, : G.shape[1] // 2], tm.test_swiglu_closed_forms),
    ("reduce indexes Y by slot, not row", moe, "unpermute_reduce",
     lambda Y, s2r, w: moe.__dict__["_orig_unpermute_reduce"](Y, np.arange(len(s2r)), w),
     tm.test_unpermute_reduce_gather_and_one_hot),
    ("ue8m0 bias 126", mxfp4, "E8M0_TABLE", np.ldexp(1.0, np.arange(256) - 126),
     tx.test_e8m0_table_matches_torch_cast),
    ("mx shared exponent with emax 3", mxfp4, "E2M1_EMAX", 3, tx.test_grid_inputs_round_trip_exactly),
    ("mx shared exponent rounds log2", mxfp4, "shared_exponent",
     lambda a: np.maximum(np.round(np.log2(np.asarray(a, np.float64))).astype(np.int64) - 2, -127),
     tx.test_grid_inputs_round_trip_exactly),
    ("mx dequantize scale per 16", mxfp4, "GROUP", 16, tx.test_hand_examples),
    ("mxfp8 shared exponent with emax 7", mxfp8, "E4M3_EMAX", 7, t8.test_grid_inputs_round_trip_exactly),
    ("mxfp8 rounds the scale exponent", mxfp8, "shared_exponent",
     lambda a: np.maximum(np.round(np.log2(np.asarray(a, np.float64))).astype(np.int64) - 8, -127),
     t8.test_codes_match_torch_e4m3fn_cast),
]


@pytest.mark.parametrize("name,mod,attr,repl,pin", MUTATIONS, ids=[m[0] for m in MUTATIONS])
def test_pin_catches_planted_mistake(monkeypatch, name, mod, attr, repl, pin):
    monkeypatch.setitem(mod.__dict__, "_orig_" + attr, getattr(mod, attr))
    monkeypatch.setattr(mod, attr, repl)
    with pytest.raises(AssertionError):
        pin()
