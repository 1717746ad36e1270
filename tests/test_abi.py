"""The C ABI without a GPU: the library loads, exports every symbol the header
declares, and host-side validation returns the documented error codes before
any launch (no compute call is made here)."""
import ctypes as C
import os
import re

import pytest

import bit_moe_amd as bm
from bit_moe_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "bitmoe.h")


def _header_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(moe_[a-z0-9_]+)\s*\(", src)))


def test_header_declares_what_binding_lists():
    assert _header_functions() == sorted(_lib.SYMBOLS)


def test_library_exports_every_declared_symbol():
    L = bm.lib()
    for name in _header_functions():
        assert hasattr(L, name), name
    assert "gfx950" in bm.version()


def test_checked_ids_build_exports_the_same_symbols_and_workspaces():
    """libbitmoe_checked.so (BITMOE_CHECK_IDS=1): the same entry points and
    workspace sizes, the first 256 bytes of the bucketing and FFN workspaces
    holding the count of bad ids."""
    C = bm.lib_checked()
    for name in _header_functions():
        assert hasattr(C, name), name
    assert "checked" in C.moe_version().decode() and "checked" not in bm.version()
    L = bm.lib()
    for T, k, E in ((1, 8, 256), (16, 8, 256), (8192, 8, 256)):
        assert C.moe_bucket_workspace_bytes(T, k, E) == L.moe_bucket_workspace_bytes(T, k, E)
    # the count's 256 bytes come before the bucketing scratch
    assert L.moe_bucket_workspace_bytes(8192, 8, 256) >= 256 + 8192 * 8 // 256
    lay = _layer()
    for mode in (bm.DECODE, bm.PREFILL):
        assert C.moe_workspace_bytes(lay, 16, mode) == L.moe_workspace_bytes(lay, 16, mode) > 256


def test_strerror_names_every_code():
    for code in (0, -1, -2, -3, -4):
        assert bm.strerror(code)
    assert "unknown" in bm.strerror(-99)


def _layer(H=256, I=512, E=8, k=2, shared=False, **kw):
    d = dict(H=H, I=I, E=E, k=k, router_w=16, gate_q=16, up_q=16, down_q=16, grid=16,
             shared_gate=16 if shared else None, shared_up=16 if shared else None,
             shared_down=16 if shared else None, layout=_lib.LAYOUT_TILED, fmt=_lib.FORMAT_2BIT)
    d.update(kw)
    return _lib.LayerStruct(d["H"], d["I"], d["E"], d["k"], d["router_w"], d["gate_q"], d["up_q"],
                            d["down_q"], d["grid"], d["shared_gate"], d["shared_up"], d["shared_down"],
                            d["layout"], d["fmt"])


@pytest.mark.parametrize("kw,code", [
    (dict(H=100), _lib.EUNSUPPORTED), (dict(I=300), _lib.EUNSUPPORTED),
    (dict(k=17, E=32), _lib.EUNSUPPORTED), (dict(k=9, E=8), _lib.EUNSUPPORTED),
    (dict(E=2000), _lib.EUNSUPPORTED), (dict(H=0), _lib.EINVAL), (dict(k=0), _lib.EINVAL),
    (dict(router_w=None), _lib.EINVAL),
])
def test_route_rejects_bad_layers(kw, code):
    L = bm.lib()
    lay = _layer(**kw)
    rc = L.moe_route(C.byref(lay), 16, 0, 4, None, 16, 16, 256, 1 << 20, None)
    assert rc == code


def test_route_argument_checks():
    L = bm.lib()
    lay = _layer()
    ref = C.byref(lay)
    assert L.moe_route(ref, 16, 0, 0, None, None, None, None, 0, None) == 0      # T = 0: no-op
    assert L.moe_route(ref, 16, 0, -1, None, 16, 16, 256, 1 << 20, None) == _lib.EINVAL
    assert L.moe_route(ref, 16, 7, 4, None, 16, 16, 256, 1 << 20, None) == _lib.EINVAL
    assert L.moe_route(ref, None, 0, 4, None, 16, 16, 256, 1 << 20, None) == _lib.EINVAL
    assert L.moe_route(ref, 8, 0, 4, None, 16, 16, 256, 1 << 20, None) == _lib.EINVAL   # misaligned x
    assert L.moe_route(ref, 16, 0, 4, None, 16, 16, None, 0, None) == _lib.EWORKSPACE
    need = L.moe_route_workspace_bytes(ref, 4, 0)
    assert need > 0
    assert L.moe_route(ref, 16, 0, 4, None, 16, 16, 256, need - 1, None) == _lib.EWORKSPACE
    assert L.moe_route(ref, 16, 0, 4, None, 16, 16, 128, need, None) == _lib.EWORKSPACE  # misaligned ws


@pytest.mark.parametrize("fn", ["moe_ffn_decode", "moe_ffn_prefill"])
def test_ffn_argument_checks(fn):
    L = bm.lib()
    f = getattr(L, fn)
    mode = 0 if fn == "moe_ffn_decode" else 1
    lay = _layer()
    ref = C.byref(lay)
    need = L.moe_workspace_bytes(ref, 4, mode)
    assert need > 0
    ok = dict(x=16, dt=1, T=4, ids=16, w=16, y=16, ws=256, n=need)

    def call(**kw):
        a = dict(ok, **kw)
        return f(ref, a["x"], a["dt"], a["T"], a["ids"], a["w"], a["y"], a["ws"], a["n"], None)
    assert call(T=0) == 0
    assert call(T=-3) == _lib.EINVAL
    assert call(dt=2) == _lib.EINVAL
    assert call(x=None) == _lib.EINVAL
    assert call(ids=None) == _lib.EINVAL
    assert call(w=None) == _lib.EINVAL
    assert call(y=None) == _lib.EINVAL
    assert call(y=8) == _lib.EINVAL
    assert call(ws=None) == _lib.EWORKSPACE
    assert call(n=need - 1) == _lib.EWORKSPACE
    assert call(T=(1 << 20) + 1) == _lib.EUNSUPPORTED
    half = _layer(shared_gate=16)                          # shared expert half-specified
    assert f(C.byref(half), 16, 1, 4, 16, 16, 16, 256, need, None) == _lib.EINVAL
    nog = _layer(gate_q=None)
    assert f(C.byref(nog), 16, 1, 4, 16, 16, 16, 256, need, None) == _lib.EINVAL
    # the FFN kernels read tiled blocks: a canonical descriptor is refused,
    # an unknown layout tag is invalid
    canon = _layer(layout=_lib.LAYOUT_CANONICAL)
    assert f(C.byref(canon), 16, 1, 4, 16, 16, 16, 256, need, None) == _lib.EUNSUPPORTED
    assert L.moe_workspace_bytes(C.byref(canon), 4, mode) == 0
    bad = _layer(layout=7)
    assert f(C.byref(bad), 16, 1, 4, 16, 16, 16, 256, need, None) == _lib.EINVAL


def test_forward_decode_checks_layout_and_router():
    L = bm.lib()
    need = L.moe_workspace_bytes(C.byref(_layer()), 4, 0)
    canon = _layer(layout=_lib.LAYOUT_CANONICAL)
    assert L.moe_forward_decode(C.byref(canon), 16, 1, 4, 16, 16, 16, 256, need, None) == _lib.EUNSUPPORTED
    norouter = _layer(router_w=None)
    assert L.moe_forward_decode(C.byref(norouter), 16, 1, 4, 16, 16, 16, 256, need, None) == _lib.EINVAL
    # routing reads only the router: a canonical descriptor routes
    rneed = L.moe_route_workspace_bytes(C.byref(canon), 4, 0)
    assert L.moe_route(C.byref(canon), 16, 0, 0, None, 16, 16, 256, rneed, None) == 0


@pytest.mark.parametrize("T", [17, 64, 200])
@pytest.mark.parametrize("x_dtype", [0, 1])
def test_forward_decode_workspace_covers_its_router(T, x_dtype):
    """Batches above the fused-router size are routed by moe_route inside
    moe_forward_decode; the decode workspace must hold that router's scratch
    for either activation dtype (bf16 from 64 tokens takes the split-K
    matrix-core router, eight partial sums per logit)."""
    L = bm.lib()
    lay = _layer(H=7168, I=2048, E=256, k=8, shared=True)
    ws = L.moe_workspace_bytes(C.byref(lay), T, 0)
    assert ws >= L.moe_route_workspace_bytes(C.byref(lay), T, x_dtype)
    if x_dtype == 1 and T >= 64:
        assert ws >= 8 * T * 256 * 4


def test_timing_event_selector_checks():
    L = bm.lib()
    assert L.moe_set_timing_events(None, None, _lib.TIME_GATEUP) == 0
    assert L.moe_set_timing_events(None, None, _lib.TIME_DOWN) == 0
    assert L.moe_set_timing_events(None, None, 2) == _lib.EINVAL
    assert L.moe_set_timing_events(16, None, 0) == _lib.EINVAL


def test_workspace_sizes_grow_with_tokens_and_shared():
    L = bm.lib()
    for mode in (0, 1):
        a = L.moe_workspace_bytes(C.byref(_layer(H=7168, I=2048, E=256, k=8)), 16, mode)
        b = L.moe_workspace_bytes(C.byref(_layer(H=7168, I=2048, E=256, k=8)), 2048, mode)
        c = L.moe_workspace_bytes(C.byref(_layer(H=7168, I=2048, E=256, k=8, shared=True)), 16, mode)
        assert 0 < a < b and a < c
        assert a % 256 == 0
    assert L.moe_workspace_bytes(C.byref(_layer()), 4, 5) == 0
    assert L.moe_workspace_bytes(C.byref(_layer(H=100)), 4, 0) == 0


def test_dequant_pack_topk_bucket_argument_checks():
    L = bm.lib()
    assert L.moe_dequant_iq2x(16, 16, 0, 16, 0, None) == 0
    assert L.moe_dequant_iq2x(16, 16, -1, 16, 0, None) == _lib.EINVAL
    assert L.moe_dequant_iq2x(16, 16, 4, 16, 3, None) == _lib.EINVAL
    assert L.moe_dequant_iq2x(None, 16, 4, 16, 0, None) == _lib.EINVAL
    assert L.moe_dequant_iq2x(16, None, 4, 16, 0, None) == _lib.EINVAL
    assert L.moe_dequant_q2k(16, 4, None, 0, None) == _lib.EINVAL
    assert L.moe_dequant_q2k(18, 4, 16, 0, None) == _lib.EINVAL          # misaligned blocks
    assert L.moe_pack_iq2x(16, 16, 1, 100, 256, None) == _lib.EUNSUPPORTED
    assert L.moe_pack_q2k(16, 16, 1, 64, 100, None) == _lib.EUNSUPPORTED
    assert L.moe_pack_bf16(16, 16, 64, 12, None) == _lib.EUNSUPPORTED
    assert L.moe_pack_iq2x(None, 16, 1, 64, 256, None) == _lib.EINVAL
    assert L.moe_topk(16, 4, 8, 9, 16, 16, None) == _lib.EUNSUPPORTED
    assert L.moe_topk(None, 4, 8, 2, 16, 16, None) == _lib.EINVAL
    assert L.moe_topk(16, 0, 8, 2, None, None, None) == 0
    assert L.moe_bucket_workspace_bytes(0, 8, 256) == 0
    assert L.moe_bucket(16, 4, 2, 8, None, 16, 16, 16, 16, 256, 256, None) == _lib.EINVAL
    big = L.moe_bucket_workspace_bytes(8192, 8, 256)
    assert big >= 64 * 256 * 4
    assert L.moe_bucket(16, 8192, 8, 256, 16, 16, 16, 16, 16, 256, big - 1, None) == _lib.EWORKSPACE


def test_noalloc_refuses_calls_beyond_its_static_scratch():
    """The allocation-free decode call checks its scratch need on the host,
    before any device work: 64 tokens at full shape with a shared expert
    need more than the static array, 16 tokens fit."""
    L = bm.lib()
    lay = _layer(H=7168, I=2048, E=256, k=8, shared=True)
    assert L.moe_workspace_bytes(C.byref(lay), 16, 0) <= _lib.STATIC_SCRATCH_BYTES
    assert L.moe_workspace_bytes(C.byref(lay), 64, 0) > _lib.STATIC_SCRATCH_BYTES
    assert L.moe_forward_decode_noalloc(C.byref(lay), 16, 1, 64, 16, 16, 16, None) == _lib.ESCRATCH
    assert L.moe_forward_decode_noalloc(C.byref(lay), 16, 1, 0, 16, 16, 16, None) == 0
    assert L.moe_forward_decode_noalloc(C.byref(lay), None, 1, 4, 16, 16, 16, None) == _lib.EINVAL
    canon = _layer(layout=_lib.LAYOUT_CANONICAL)
    assert L.moe_forward_decode_noalloc(C.byref(canon), 16, 1, 4, 16, 16, 16, None) == _lib.EUNSUPPORTED
    assert "static" in bm.strerror(_lib.ESCRATCH)


def test_quantize_argument_checks():
    L = bm.lib()
    assert L.moe_quantize_iq2x(16, 16, 0, 16, None) == 0
    assert L.moe_quantize_iq2x(16, 16, -1, 16, None) == _lib.EINVAL
    assert L.moe_quantize_iq2x(None, 16, 4, 16, None) == _lib.EINVAL
    assert L.moe_quantize_iq2x(16, None, 4, 16, None) == _lib.EINVAL
    assert L.moe_quantize_iq2x(8, 16, 4, 16, None) == _lib.EINVAL       # misaligned weights
    assert L.moe_quantize_q2k(16, 4, None, None) == _lib.EINVAL
    assert L.moe_quantize_q2k(16, -2, 16, None) == _lib.EINVAL
    assert L.moe_quantize_q2k(16, 0, None, None) == 0


def test_format_tag_and_mxfp4_entry_points():
    """The layer's format tag: an unknown tag is invalid; a 2-bit layer needs
    the codebook, an MXFP4 layer does not (a T = 0 call passes every check
    and queues nothing).  MXFP4 dequant / pack argument checks, and the cache
    pool of an MXFP4 layer (17 bytes per 32 weights per slab)."""
    L = bm.lib()
    x = y = ids = w = 16
    for f in (L.moe_ffn_decode, L.moe_ffn_prefill):
        bad = _layer(fmt=7)
        assert f(C.byref(bad), x, 1, 4, ids, w, y, 256, 1 << 20, None) == _lib.EINVAL
        assert L.moe_workspace_bytes(C.byref(bad), 4, 0) == 0
        nog = _layer(grid=None)
        assert f(C.byref(nog), x, 1, 4, ids, w, y, 256, 1 << 20, None) == _lib.EINVAL
        mx = _layer(grid=None, fmt=_lib.FORMAT_MXFP4)
        assert f(C.byref(mx), x, 1, 0, ids, w, y, None, 0, None) == 0
        assert L.moe_workspace_bytes(C.byref(mx), 4, 0) > 0
        assert f(C.byref(mx), x, 1, 4, ids, w, y, None, 0, None) == _lib.EWORKSPACE
    assert L.moe_dequant_mxfp4(16, -1, 16, 0, None) == _lib.EINVAL
    assert L.moe_dequant_mxfp4(16, 4, 16, 2, None) == _lib.EINVAL
    assert L.moe_dequant_mxfp4(16, 4, 8, 0, None) == _lib.EINVAL            # out not 16-byte aligned
    assert L.moe_dequant_mxfp4(None, 4, 16, 0, None) == _lib.EINVAL
    assert L.moe_dequant_mxfp4(None, 0, None, 0, None) == 0
    assert L.moe_pack_mxfp4(16, 16, 2, 64, 32, None) == _lib.EUNSUPPORTED   # K not a multiple of 256
    assert L.moe_pack_mxfp4(16, 16, 2, 100, 256, None) == _lib.EUNSUPPORTED
    assert L.moe_pack_mxfp4(16, 8, 2, 64, 256, None) == _lib.EINVAL          # dst not 16-byte aligned
    assert L.moe_pack_mxfp4(None, None, 0, 64, 256, None) == 0
    mx = _layer(H=7168, I=2048, E=256, k=8, grid=None, fmt=_lib.FORMAT_MXFP4)
    slab = 2 * 2048 * 7168 // 32 * 17 + 7168 * 2048 // 32 * 17
    assert L.moe_cache_pool_bytes(C.byref(mx), 24) == 3 * 256 + 24 * slab
    two = _layer(H=7168, I=2048, E=256, k=8)
    assert L.moe_cache_pool_bytes(C.byref(two), 24) == 3 * 256 + 24 * (2 * 2048 * 28 * 66 + 7168 * 8 * 84)


def test_quantize_mxfp4_argument_checks():
    L = bm.lib()
    assert L.moe_quantize_mxfp4(16, -1, 16, None) == _lib.EINVAL
    assert L.moe_quantize_mxfp4(None, 0, None, None) == 0
    assert L.moe_quantize_mxfp4(None, 4, 16, None) == _lib.EINVAL
    assert L.moe_quantize_mxfp4(8, 4, 16, None) == _lib.EINVAL                # w not 16-byte aligned
