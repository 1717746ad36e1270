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


def test_strerror_names_every_code():
    for code in (0, -1, -2, -3, -4):
        assert bm.strerror(code)
    assert "unknown" in bm.strerror(-99)


def _layer(H=256, I=512, E=8, k=2, shared=False, **kw):
    d = dict(H=H, I=I, E=E, k=k, router_w=16, gate_q=16, up_q=16, down_q=16, grid=16,
             shared_gate=16 if shared else None, shared_up=16 if shared else None,
             shared_down=16 if shared else None)
    d.update(kw)
    return _lib.LayerStruct(d["H"], d["I"], d["E"], d["k"], d["router_w"], d["gate_q"], d["up_q"],
                            d["down_q"], d["grid"], d["shared_gate"], d["shared_up"], d["shared_down"])


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
