"""CPU-only checks of the C ABI library: it loads, exports every symbol the header declares,
and rejects bad arguments on the host before any HIP call (so no GPU is needed)."""
import ctypes
import os
import re

import pytest

from nvfp4_block_scaled_moe_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "nvfp4moe.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    names = re.findall(r"\b(?:nvfp4moe_status|size_t|const char\*|int)\s+(\w+)\s*\(", text)
    return sorted(set(names))


def test_header_declares_the_calls():
    names = declared_functions()
    for want in ["nvfp4_quantize", "moe_route_permute", "moe_grouped_gemm_nvfp4",
                 "moe_unpermute_reduce", "act_fp8_e4m3_roundtrip", "nvfp4moe_last_error",
                 "nvfp4_weights_tile"]:
        assert want in names


def test_library_exports_every_declared_symbol():
    lib = _lib.load()
    names = declared_functions()
    assert set(names) == set(_lib.SIGNATURES), "binding signatures out of sync with the header"
    for n in names:
        assert hasattr(lib, n)
    assert lib.nvfp4moe_abi_version() == 302


FAKE = ctypes.c_void_p(1 << 20)      # aligned, never dereferenced: validation fails first
MISALIGNED = ctypes.c_void_p((1 << 20) + 2)


def _err(st):
    return st, _lib.load().nvfp4moe_last_error().decode()


def test_quantize_rejects_bad_arguments():
    lib = _lib.load()
    st, msg = _err(lib.nvfp4_quantize(None, _lib.F32, 1, 4, 32, None, None, 0, FAKE, FAKE, FAKE, FAKE, 1 << 20, None))
    assert st == _lib.ERR_INVALID_ARG and "null" in msg
    st, msg = _err(lib.nvfp4_quantize(FAKE, _lib.F32, 1, 4, 48, None, None, 0, FAKE, FAKE, FAKE, FAKE, 1 << 20, None))
    assert st == _lib.ERR_INVALID_ARG and "C % 32" in msg
    st, _ = _err(lib.nvfp4_quantize(FAKE, 7, 1, 4, 32, None, None, 0, FAKE, FAKE, FAKE, FAKE, 1 << 20, None))
    assert st == _lib.ERR_INVALID_ARG
    st, _ = _err(lib.nvfp4_quantize(MISALIGNED, _lib.F32, 1, 4, 32, None, None, 0, FAKE, FAKE, FAKE, FAKE, 1 << 20, None))
    assert st == _lib.ERR_INVALID_ARG
    need = lib.nvfp4_quantize_workspace_size(1, 4, 32)
    st, msg = _err(lib.nvfp4_quantize(FAKE, _lib.F32, 1, 4, 32, None, None, 0, FAKE, FAKE, FAKE, FAKE, need - 1, None))
    assert st == _lib.ERR_WORKSPACE and "workspace" in msg


def test_quantize_tiled_layout_argument_checks():
    lib = _lib.load()
    call = lambda R, layout, sc=FAKE: _err(lib.nvfp4_quantize(FAKE, _lib.F32, 1, R, 64, None, None, layout, FAKE, sc,
                                                             FAKE, FAKE, 1 << 20, None))
    st, msg = call(24, _lib.LAYOUT_TILED)
    assert st == _lib.ERR_INVALID_ARG and "R % 16" in msg
    st, msg = call(32, 2)
    assert st == _lib.ERR_INVALID_ARG and "layout" in msg
    st, msg = call(32, _lib.LAYOUT_TILED, ctypes.c_void_p((1 << 20) + 2))
    assert st == _lib.ERR_INVALID_ARG and "16-byte" in msg
    st, _ = _err(lib.nvfp4_quantize_noalloc(FAKE, _lib.F32, 1, 24, 64, None, None, _lib.LAYOUT_TILED, FAKE, FAKE,
                                            FAKE, None))
    assert st == _lib.ERR_INVALID_ARG


def test_quantize_noalloc_rejects_bad_arguments():
    """Argument checks of the no-allocation quantize: the same as nvfp4_quantize, plus a batch
    whose amax partials exceed the 64 KiB scratch (host-side, before any HIP call)."""
    lib = _lib.load()
    st, msg = _err(lib.nvfp4_quantize_noalloc(None, _lib.F32, 1, 4, 32, None, None, 0, FAKE, FAKE, FAKE, None))
    assert st == _lib.ERR_INVALID_ARG and "null" in msg
    st, msg = _err(lib.nvfp4_quantize_noalloc(FAKE, _lib.F32, 1, 4, 48, None, None, 0, FAKE, FAKE, FAKE, None))
    assert st == _lib.ERR_INVALID_ARG and "C % 32" in msg
    st, _ = _err(lib.nvfp4_quantize_noalloc(MISALIGNED, _lib.F32, 1, 4, 32, None, None, 0, FAKE, FAKE, FAKE, None))
    assert st == _lib.ERR_INVALID_ARG
    assert lib.nvfp4_quantize_workspace_size(16, 4096, 4096) == 65536    # fits exactly
    assert lib.nvfp4_quantize_workspace_size(32, 4096, 4096) > 65536
    st, msg = _err(lib.nvfp4_quantize_noalloc(FAKE, _lib.F32, 32, 4096, 4096, None, None, 0, FAKE, FAKE, FAKE, None))
    assert st == _lib.ERR_WORKSPACE and "65536" in msg


def test_route_permute_rejects_bad_arguments():
    lib = _lib.load()
    args = lambda T, E, k: (FAKE, T, E, k, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None, 0, None)
    for T, E, k in [(0, 8, 2), (4, 8, 9), (4, 8, 0), (4, 2048, 8), (4, 256, 65), (1 << 22, 256, 8)]:
        st, _ = _err(lib.moe_route_permute(*args(T, E, k)))
        assert st == _lib.ERR_INVALID_ARG, (T, E, k)


def test_mxfp4_swiglu_q_argument_checks():
    lib = _lib.load()

    def call(hp=FAKE, hs=FAKE, Nw=256, K=256, ws_bytes=1 << 30):
        return lib.moe_grouped_gemm_mxfp4_swiglu_q(FAKE, FAKE, 16, None, 1, FAKE, FAKE, FAKE, FAKE, FAKE, 8, 16,
                                                   Nw, K, hp, hs, FAKE, ws_bytes, None)
    for kw in [dict(hp=None), dict(hs=None), dict(hp=MISALIGNED), dict(hs=ctypes.c_void_p((1 << 20) + 2)),
               dict(K=48)]:
        st, _ = _err(call(**kw))
        assert st == _lib.ERR_INVALID_ARG, kw
    st, _ = _err(call(Nw=384))
    assert st == _lib.ERR_UNSUPPORTED
    st, _ = _err(call(ws_bytes=8))
    assert st == _lib.ERR_WORKSPACE


def test_mxfp8_argument_checks_and_sizes():
    lib = _lib.load()

    def gemm(**kw):
        a = dict(epi=_lib.EPI_NONE, a=FAKE, a_rows=16, E=8, rows=16, Nw=256, K=256, ws_bytes=1 << 30)
        a.update(kw)
        return lib.moe_grouped_gemm_mxfp8(a["epi"], a["a"], FAKE, a["a_rows"], None, 1, FAKE, FAKE, FAKE, FAKE, FAKE,
                                          a["E"], a["rows"], a["Nw"], a["K"], FAKE, _lib.F32, None, FAKE,
                                          a["ws_bytes"], None)
    for kw in [dict(epi=4), dict(a=None), dict(E=0), dict(rows=0), dict(K=48), dict(a=MISALIGNED)]:
        st, _ = _err(gemm(**kw))
        assert st == _lib.ERR_INVALID_ARG, kw
    st, _ = _err(gemm(Nw=384))
    assert st == _lib.ERR_UNSUPPORTED
    st, _ = _err(gemm(ws_bytes=8))
    assert st == _lib.ERR_WORKSPACE
    st, _ = _err(lib.mxfp8_quantize(FAKE, _lib.F32, 4, 48, FAKE, FAKE, None))
    assert st == _lib.ERR_INVALID_ARG
    assert lib.mxfp8_tiled_codes_bytes(32, 256) == 2 * 2 * 2048
    assert lib.mxfp8_tiled_codes_bytes(30, 256) == 0
    # 64-row m-tiles: M = 512, N = 2048 has 9 x 8 tiles (host bound) -> K split in 4
    assert lib.moe_grouped_gemm_mxfp8_workspace_size(512, 1, 2048, 6144) >= 4 * 512 * 2048 * 4


def test_route_permute_workspace():
    """The permutation's workspace holds per-chunk expert counts (chunks of >= 2048 slots, at
    most 64 chunks); a call with less is rejected before any HIP call."""
    lib = _lib.load()
    assert lib.moe_route_permute_workspace_size(8192, 256, 8) == 32 * 256 * 4
    assert lib.moe_route_permute_workspace_size(1, 256, 8) == 256 * 4
    assert lib.moe_route_permute_workspace_size(1 << 20, 64, 16) == 64 * 64 * 4
    assert lib.moe_route_permute_workspace_size(0, 256, 8) == 0
    assert lib.moe_route_permute_workspace_size(4, 8, 9) == 0
    need = lib.moe_route_permute_workspace_size(512, 256, 8)
    for ws, nbytes in [(None, 0), (FAKE, need - 1)]:
        st, msg = _err(lib.moe_route_permute(FAKE, 512, 256, 8, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE,
                                             ws, nbytes, None))
        assert st == _lib.ERR_WORKSPACE and "workspace" in msg


def _gemm(lib, mode=_lib.W4A16, epi=_lib.EPI_SWIGLU, a=FAKE, a_scales=None, a_g=None, a_rows=16,
          gidx=None, gdiv=1, E=8, rows=16, Nw=64, K=64, out_dtype=_lib.BF16, ws=FAKE, ws_bytes=1 << 30):
    return lib.moe_grouped_gemm_nvfp4(mode, epi, a, a_scales, a_g, a_rows, gidx, gdiv, FAKE, FAKE, FAKE,
                                      FAKE, FAKE, FAKE, E, rows, Nw, K, FAKE, out_dtype, None, ws,
                                      ws_bytes, None)


def test_grouped_gemm_rejects_bad_arguments():
    lib = _lib.load()
    bad = [
        dict(mode=5), dict(epi=3), dict(out_dtype=9), dict(a=None), dict(mode=_lib.W4A4),
        dict(E=0), dict(E=2000), dict(rows=0), dict(Nw=48), dict(Nw=16), dict(K=40), dict(K=0),
        dict(a_rows=8), dict(gidx=FAKE, gdiv=0), dict(a=MISALIGNED), dict(rows=1 << 26, a_rows=1 << 26, K=64, Nw=64),
    ]
    for kw in bad:
        st, _ = _err(_gemm(lib, **kw))
        assert st == _lib.ERR_INVALID_ARG, kw
    need = lib.moe_grouped_gemm_workspace_size(_lib.W4A16, 16, 16, 8, 64, 64)
    assert need >= 16 * 64 * 2
    st, _ = _err(_gemm(lib, ws_bytes=need - 1))
    assert st == _lib.ERR_WORKSPACE


def test_grouped_gemm_workspace_follows_the_path(monkeypatch):
    """The m-tiled path needs f16 activations (also for W4A4) and its m-tile schedule; the
    size query and the call pick the path by the same rule, and a forced MFMA path that
    cannot run the shape is refused before any work is queued."""
    lib = _lib.load()
    ws = lib.moe_grouped_gemm_workspace_size
    monkeypatch.delenv("NVFP4MOE_FORCE_PATH", raising=False)
    assert ws(_lib.W4A4, 512, 512, 64, 256, 256) == 0                 # 8 rows/expert: streaming
    big = ws(_lib.W4A4, 8192, 8192, 64, 256, 256)                      # 128 rows/expert: MFMA
    assert big >= 8192 * 256 * 2 + 8192 * 4 + 2 * (8192 // 128 + 64) * 4
    assert ws(_lib.W4A16, 8192, 8192, 64, 256, 256) == big
    assert ws(_lib.W4A4, 8192, 8192, 64, 160, 256) == 0                # Nw % 256 != 0: streaming
    monkeypatch.setenv("NVFP4MOE_FORCE_PATH", "mfma")
    assert ws(_lib.W4A4, 512, 512, 64, 256, 256) > 512 * 256 * 2
    st, msg = _err(_gemm(lib, Nw=96))
    assert st == _lib.ERR_UNSUPPORTED and "256" in msg
    monkeypatch.setenv("NVFP4MOE_FORCE_PATH", "stream")
    assert ws(_lib.W4A4, 8192, 8192, 64, 256, 256) == 0


def test_weights_tile_sizes_and_argument_checks():
    lib = _lib.load()
    # closed forms: (R/16) * ceil(C/128) KB of codes, (R/16) * ceil(C/1024) KB of scales
    assert lib.nvfp4_tiled_codes_bytes(4096, 7168) == 256 * 56 * 1024
    assert lib.nvfp4_tiled_scales_bytes(4096, 7168) == 256 * 7 * 1024
    assert lib.nvfp4_tiled_codes_bytes(16, 160) == 2 * 1024
    assert lib.nvfp4_tiled_scales_bytes(48, 1056) == 3 * 2 * 1024
    for R, C in [(8, 64), (24, 64), (16, 48), (16, 0)]:
        assert lib.nvfp4_tiled_codes_bytes(R, C) == 0 and lib.nvfp4_tiled_scales_bytes(R, C) == 0
    ok = (FAKE, FAKE, 1, 32, 64, FAKE, FAKE, None)
    bad = [(None,) + ok[1:], ok[:2] + (0,) + ok[3:], ok[:3] + (24,) + ok[4:], ok[:4] + (48,) + ok[5:],
           ok[:5] + (MISALIGNED,) + ok[6:], ok[:6] + (ctypes.c_void_p((1 << 20) + 2),) + ok[7:]]
    for args in bad:
        st, _ = _err(lib.nvfp4_weights_tile(*args))
        assert st == _lib.ERR_INVALID_ARG, args


def test_unpermute_reduce_and_fp8_reject_bad_arguments():
    lib = _lib.load()
    assert lib.moe_unpermute_reduce(FAKE, _lib.F32, FAKE, FAKE, 4, 2, 12, FAKE, None) == _lib.ERR_INVALID_ARG
    assert lib.moe_unpermute_reduce(FAKE, _lib.F32, FAKE, FAKE, 0, 2, 16, FAKE, None) == _lib.ERR_INVALID_ARG
    assert lib.moe_unpermute_reduce(None, _lib.F32, FAKE, FAKE, 4, 2, 16, FAKE, None) == _lib.ERR_INVALID_ARG
    assert lib.act_fp8_e4m3_roundtrip(FAKE, 12, FAKE, FAKE, 1 << 20, None) == _lib.ERR_INVALID_ARG
    assert lib.act_fp8_e4m3_roundtrip(FAKE, 64, FAKE, FAKE, 0, None) == _lib.ERR_WORKSPACE


def test_last_error_is_thread_local_and_cleared():
    import threading
    lib = _lib.load()
    lib.moe_route_permute(*(FAKE, 0, 8, 2, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None, 0, None))
    assert lib.nvfp4moe_last_error()
    seen = []
    th = threading.Thread(target=lambda: seen.append(lib.nvfp4moe_last_error()))
    th.start()
    th.join()
    assert seen == [b""]



def _mx_gemm(lib, epi=_lib.EPI_NONE, a=FAKE, a_rows=16, gidx=None, gdiv=1, E=8, rows=16, Nw=256, K=256,
             out_dtype=_lib.F32, ws=FAKE, ws_bytes=1 << 30):
    return lib.moe_grouped_gemm_mxfp4(epi, a, FAKE, a_rows, gidx, gdiv, FAKE, FAKE, FAKE, FAKE, FAKE, E, rows,
                                      Nw, K, FAKE, out_dtype, None, ws, ws_bytes, None)


def test_mxfp4_argument_checks_and_sizes():
    """The MXFP4 calls validate before queuing anything; sizes follow the closed forms."""
    lib = _lib.load()
    for R, C in [(16, 32), (32, 2048), (48, 2080), (16, 4096)]:
        assert lib.mxfp4_tiled_scales_bytes(R, C) == (R // 16) * -(-C // 2048) * 1024
    assert lib.mxfp4_tiled_scales_bytes(15, 64) == 0 and lib.mxfp4_tiled_scales_bytes(16, 48) == 0
    for args in [(FAKE, _lib.F32, 4, 48), (FAKE, _lib.F32, 0, 64), (FAKE, 7, 4, 64), (None, _lib.F32, 4, 64),
                 (MISALIGNED, _lib.BF16, 4, 64)]:
        st, _ = _err(lib.mxfp4_quantize(*args, FAKE, FAKE, None))
        assert st == _lib.ERR_INVALID_ARG, args
    st, _ = _err(lib.mxfp4_weights_tile(FAKE, FAKE, 1, 24, 64, FAKE, FAKE, None))
    assert st == _lib.ERR_INVALID_ARG
    bad = [dict(epi=4), dict(out_dtype=5), dict(a=None), dict(E=0), dict(E=2000), dict(rows=0), dict(K=48),
           dict(K=0), dict(a_rows=8), dict(gidx=FAKE, gdiv=0), dict(a=MISALIGNED)]
    for kw in bad:
        st, _ = _err(_mx_gemm(lib, **kw))
        assert st == _lib.ERR_INVALID_ARG, kw
    st, msg = _err(_mx_gemm(lib, Nw=384))
    assert st == _lib.ERR_UNSUPPORTED and "256" in msg
    need = lib.moe_grouped_gemm_mxfp4_workspace_size(16, 8, 256, 256)
    assert need >= 2 * (1 + 8) * 4
    # a grid under one workgroup per CU splits K: M = 512, N = 2048, K = 6144 (48 chunks) has
    # 5 x 8 tiles (host bound) -> 7 slices of 7 chunks, fp32 partial sums [7, 512, 2048]
    assert lib.moe_grouped_gemm_mxfp4_workspace_size(512, 1, 2048, 6144) >= 7 * 512 * 2048 * 4
    assert lib.moe_grouped_gemm_mxfp4_workspace_size(65536, 256, 4096, 7168) < 1 << 20   # no split
    assert lib.moe_grouped_gemm_mxfp4_workspace_size(0, 8, 256, 64) == 0
    st, _ = _err(_mx_gemm(lib, ws_bytes=need - 1))
    assert st == _lib.ERR_WORKSPACE


def test_dispatch_rejects_bad_arguments_and_sizes():
    """moe_dispatch_w4a16: host-side checks (null outputs, H % 32, fp8 flag, alignment,
    workspace) and its size queries; the prepared-row GEMM mode shares the GEMM's checks."""
    lib = _lib.load()
    T, E, k, H = 2, 8, 2, 64
    ws = lib.moe_dispatch_w4a16_workspace_size(T, E, k, H, 0)

    def call(x=FAKE, h=H, fp8=0, x_prep=FAKE, wsp=FAKE, nbytes=1 << 20, ids=FAKE):
        return _err(lib.moe_dispatch_w4a16(FAKE, x, T, E, k, h, fp8, ids, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE,
                                           x_prep, wsp, nbytes, None))
    st, msg = call(ids=None)
    assert st == _lib.ERR_INVALID_ARG and "null" in msg
    st, msg = call(x_prep=None)
    assert st == _lib.ERR_INVALID_ARG and "null" in msg
    st, msg = call(h=48)
    assert st == _lib.ERR_INVALID_ARG and "H % 32" in msg
    st, msg = call(fp8=2)
    assert st == _lib.ERR_INVALID_ARG and "fp8_act" in msg
    st, msg = call(x=MISALIGNED)
    assert st == _lib.ERR_INVALID_ARG and "16-byte" in msg
    need_fp8 = lib.moe_dispatch_w4a16_workspace_size(T, E, k, H, 1)
    assert need_fp8 > ws
    st, msg = _err(lib.moe_dispatch_w4a16(FAKE, FAKE, T, E, k, H, 1, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE,
                                          FAKE, need_fp8 - 1, None))
    assert st == _lib.ERR_WORKSPACE and "workspace" in msg
    # sizes: f16 rows padded to whole 128-column chunks, then the int32 exponents (256-byte units)
    assert lib.moe_prepared_act_bytes(3, 160) == 256 * ((3 * 256 * 2 + 255) // 256) + 256
    assert lib.moe_prepared_act_bytes(3, 48) == 0 and lib.moe_prepared_act_bytes(0, 64) == 0
    assert lib.moe_dispatch_w4a16_workspace_size(T, E, k, 48, 0) == 0
    st, msg = _err(lib.moe_grouped_gemm_nvfp4(3, 0, FAKE, None, None, T, None, 1, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE,
                                              E, T, 64, H, FAKE, _lib.F32, None, FAKE, 1 << 20, None))
    assert st == _lib.ERR_INVALID_ARG and "mode" in msg
