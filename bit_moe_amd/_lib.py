"""ctypes binding of libbitmoe.so: argument marshalling only.

Every step of the layer runs in the library's HIP kernels; this module maps
torch tensors to device pointers and the current HIP stream, allocates
outputs and workspaces with torch, and turns error codes into exceptions.
There is no fallback: if the library is missing, loading it raises.
"""
from __future__ import annotations

import ctypes as C
import os
from typing import Optional

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libbitmoe.so")
LIB_CHECKED_PATH = os.path.join(HERE, "libbitmoe_checked.so")    # built with BITMOE_CHECK_IDS = 1

F32, BF16 = 0, 1
DECODE, PREFILL = 0, 1
LAYOUT_CANONICAL, LAYOUT_TILED = 0, 1
FORMAT_2BIT, FORMAT_MXFP4 = 0, 1
TIME_GATEUP, TIME_DOWN = 0, 1
EINVAL, EUNSUPPORTED, EWORKSPACE, EHIP, ESCRATCH = -1, -2, -3, -4, -5
STATIC_SCRATCH_BYTES = 16 << 20

# every symbol declared in include/bitmoe.h
SYMBOLS = [
    "moe_route_workspace_bytes", "moe_route", "moe_topk", "moe_bucket_workspace_bytes",
    "moe_bucket", "moe_workspace_bytes", "moe_ffn_decode", "moe_forward_decode", "moe_forward_decode_noalloc",
    "moe_ffn_prefill",
    "moe_dequant_iq2x", "moe_dequant_q2k", "moe_dequant_mxfp4", "moe_quantize_iq2x", "moe_quantize_q2k",
    "moe_quantize_mxfp4",
    "moe_pack_iq2x", "moe_pack_q2k", "moe_pack_bf16", "moe_pack_mxfp4",
    "moe_set_timing_events", "moe_strerror", "moe_version",
    "moe_cache_pool_bytes", "moe_cache_create", "moe_cache_layer", "moe_cache_map", "moe_cache_stats",
    "moe_cache_destroy",
]


class LayerStruct(C.Structure):
    _fields_ = [("H", C.c_int32), ("I", C.c_int32), ("E", C.c_int32), ("k", C.c_int32),
                ("router_w", C.c_void_p), ("gate_q", C.c_void_p), ("up_q", C.c_void_p),
                ("down_q", C.c_void_p), ("grid", C.c_void_p), ("shared_gate", C.c_void_p),
                ("shared_up", C.c_void_p), ("shared_down", C.c_void_p), ("layout", C.c_int32),
                ("format", C.c_int32)]


_lib = None
_lib_checked = None


class BitMoEError(RuntimeError):
    def __init__(self, code: int, where: str):
        self.code = code
        super().__init__(f"{where}: {strerror(code)} (code {code})")


def lib() -> C.CDLL:
    """Load libbitmoe.so (built in-tree by bit_moe_amd.build)."""
    global _lib
    if _lib is None:
        _lib = _load(LIB_PATH)
    return _lib


def lib_checked() -> C.CDLL:
    """Load libbitmoe_checked.so: the same library built with
    BITMOE_CHECK_IDS = 1, whose FFN and bucketing calls write the count of
    the caller's routing ids outside [0, E) into the first int32 of their
    workspace."""
    global _lib_checked
    if _lib_checked is None:
        _lib_checked = _load(LIB_CHECKED_PATH)
    return _lib_checked


def _load(path: str) -> C.CDLL:
    if not os.path.exists(path):
        raise ImportError(f"{path} is not built; run `python -m bit_moe_amd.build`")
    L = C.CDLL(path)
    P, I, I64, SZ = C.c_void_p, C.c_int, C.c_int64, C.c_size_t
    LP = C.POINTER(LayerStruct)
    sig = {
        "moe_route_workspace_bytes": ([LP, I, I], SZ),
        "moe_route": ([LP, P, I, I, P, P, P, P, SZ, P], I),
        "moe_topk": ([P, I, I, I, P, P, P], I),
        "moe_bucket_workspace_bytes": ([I, I, I], SZ),
        "moe_bucket": ([P, I, I, I, P, P, P, P, P, P, SZ, P], I),
        "moe_workspace_bytes": ([LP, I, I], SZ),
        "moe_ffn_decode": ([LP, P, I, I, P, P, P, P, SZ, P], I),
        "moe_ffn_prefill": ([LP, P, I, I, P, P, P, P, SZ, P], I),
        "moe_forward_decode": ([LP, P, I, I, P, P, P, P, SZ, P], I),
        "moe_forward_decode_noalloc": ([LP, P, I, I, P, P, P, P], I),
        "moe_dequant_iq2x": ([P, P, I64, P, I, P], I),
        "moe_dequant_q2k": ([P, I64, P, I, P], I),
        "moe_dequant_mxfp4": ([P, I64, P, I, P], I),
        "moe_quantize_iq2x": ([P, P, I64, P, P], I),
        "moe_quantize_q2k": ([P, I64, P, P], I),
        "moe_quantize_mxfp4": ([P, I64, P, P], I),
        "moe_pack_iq2x": ([P, P, I, I, I, P], I),
        "moe_pack_q2k": ([P, P, I, I, I, P], I),
        "moe_pack_bf16": ([P, P, I, I, P], I),
        "moe_pack_mxfp4": ([P, P, I, I, I, P], I),
        "moe_set_timing_events": ([P, P, I], I),
        "moe_strerror": ([I], C.c_char_p),
        "moe_cache_pool_bytes": ([LP, I], SZ),
        "moe_cache_create": ([LP, P, P, P, I, P, SZ, C.POINTER(C.c_void_p)], I),
        "moe_cache_layer": ([P, LP], I),
        "moe_cache_map": ([P, P, I, P, P, P], I),
        "moe_cache_stats": ([P, C.POINTER(C.c_int64), C.POINTER(C.c_int64), P], I),
        "moe_cache_destroy": ([P], I),
        "moe_version": ([], C.c_char_p),
    }
    for name, (args, res) in sig.items():
        fn = getattr(L, name)
        fn.argtypes, fn.restype = args, res
    return L


def set_timing_events(start=None, stop=None, which=TIME_GATEUP) -> None:
    """Record torch.cuda.Event objects around one kernel (TIME_GATEUP: the
    routed gate/up kernel, TIME_DOWN: the routed down kernel) of the
    following FFN calls from this thread (None, None turns it off)."""
    sp = start.cuda_event if start is not None else None
    tp = stop.cuda_event if stop is not None else None
    _check(lib().moe_set_timing_events(sp, tp, which), "moe_set_timing_events")


def strerror(code: int) -> str:
    return lib().moe_strerror(int(code)).decode()


def version() -> str:
    return lib().moe_version().decode()


def _check(rc: int, where: str) -> None:
    if rc != 0:
        raise BitMoEError(rc, where)


# ---------------------------------------------------------------------------
# torch-facing helpers
# ---------------------------------------------------------------------------

def _torch():
    import torch
    return torch


def _ptr(t) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _stream(stream=None) -> Optional[int]:
    torch = _torch()
    s = torch.cuda.current_stream() if stream is None else stream
    return s.cuda_stream


def _x_dtype(x) -> int:
    torch = _torch()
    if x.dtype == torch.float32:
        return F32
    if x.dtype == torch.bfloat16:
        return BF16
    raise TypeError("activations must be float32 or bfloat16")


def _dev_check(*ts):
    for t in ts:
        if t is not None and (not t.is_cuda or not t.is_contiguous()):
            raise ValueError("tensors must be contiguous and on the GPU")


def _workspace(nbytes: int, device):
    torch = _torch()
    return torch.empty(max(int(nbytes), 256), dtype=torch.uint8, device=device)


class Layer:
    """A routed-MoE layer whose weights live in torch device tensors, in the
    tiled layout (moe_pack_* output).  fmt: FORMAT_2BIT (IQ2X gate/up, Q2K
    down, grid required) or FORMAT_MXFP4 (grid may be None)."""

    def __init__(self, H, I, E, k, router_w, gate_q, up_q, down_q, grid, shared=None, fmt=FORMAT_2BIT):
        _dev_check(router_w, gate_q, up_q, down_q, grid)
        self.H, self.I, self.E, self.k = H, I, E, k
        self.fmt = fmt
        self.tensors = [t for t in (router_w, gate_q, up_q, down_q, grid) if t is not None]
        sg = su = sd = None
        if shared is not None:
            sg, su, sd = shared
            _dev_check(sg, su, sd)
            self.tensors += [sg, su, sd]
        self.has_shared = shared is not None
        self.s = LayerStruct(H, I, E, k, _ptr(router_w), _ptr(gate_q), _ptr(up_q), _ptr(down_q),
                             _ptr(grid), _ptr(sg), _ptr(su), _ptr(sd), LAYOUT_TILED, fmt)

    @property
    def ref(self):
        return C.byref(self.s)


def route_workspace_bytes(layer: Layer, T: int, x_dtype: int) -> int:
    return int(lib().moe_route_workspace_bytes(layer.ref, T, x_dtype))


def workspace_bytes(layer: Layer, T: int, mode: int) -> int:
    return int(lib().moe_workspace_bytes(layer.ref, T, mode))


def route(layer: Layer, x, logits=None, ids=None, w=None, ws=None, stream=None):
    """Router logits + top-k + renormalised softmax. Returns (ids, w)."""
    torch = _torch()
    T = x.shape[0]
    xd = _x_dtype(x)
    if ids is None:
        ids = torch.empty((T, layer.k), dtype=torch.int32, device=x.device)
    if w is None:
        w = torch.empty((T, layer.k), dtype=torch.float32, device=x.device)
    need = route_workspace_bytes(layer, T, xd)
    if ws is None:
        ws = _workspace(need, x.device)
    _dev_check(x, logits, ids, w, ws)
    _check(lib().moe_route(layer.ref, _ptr(x), xd, T, _ptr(logits), _ptr(ids), _ptr(w), _ptr(ws),
                           ws.numel(), _stream(stream)), "moe_route")
    return ids, w


def topk(logits, k: int, ids=None, w=None, stream=None):
    torch = _torch()
    T, E = logits.shape
    if ids is None:
        ids = torch.empty((T, k), dtype=torch.int32, device=logits.device)
    if w is None:
        w = torch.empty((T, k), dtype=torch.float32, device=logits.device)
    _dev_check(logits, ids, w)
    _check(lib().moe_topk(_ptr(logits), T, E, k, _ptr(ids), _ptr(w), _stream(stream)), "moe_topk")
    return ids, w


def bucket(ids, E: int, stream=None, library=None):
    """Returns (counts, offsets, perm, active, n_active) int32 device tensors
    (library: lib() by default, or lib_checked())."""
    L = library or lib()
    torch = _torch()
    T, k = ids.shape
    dev = ids.device
    counts = torch.empty(E, dtype=torch.int32, device=dev)
    offsets = torch.empty(E + 1, dtype=torch.int32, device=dev)
    perm = torch.empty(max(T * k, 1), dtype=torch.int32, device=dev)
    active = torch.empty(E, dtype=torch.int32, device=dev)
    n_active = torch.empty(1, dtype=torch.int32, device=dev)
    ws = _workspace(L.moe_bucket_workspace_bytes(T, k, E), dev)
    _dev_check(ids)
    _check(L.moe_bucket(_ptr(ids), T, k, E, _ptr(counts), _ptr(offsets), _ptr(perm), _ptr(active),
                        _ptr(n_active), _ptr(ws), ws.numel(), _stream(stream)), "moe_bucket")
    return counts, offsets, perm[:T * k], active, n_active


def _ffn(fn, name, mode, layer: Layer, x, ids, w, y=None, ws=None, stream=None):
    torch = _torch()
    T = x.shape[0]
    if y is None:
        y = torch.empty((T, layer.H), dtype=torch.float32, device=x.device)
    if ws is None:
        ws = _workspace(workspace_bytes(layer, T, mode), x.device)
    _dev_check(x, ids, w, y, ws)
    _check(fn(layer.ref, _ptr(x), _x_dtype(x), T, _ptr(ids), _ptr(w), _ptr(y), _ptr(ws), ws.numel(),
              _stream(stream)), name)
    return y


def ffn_decode(layer, x, ids, w, y=None, ws=None, stream=None, library=None):
    """Decode FFN (moe_ffn_decode); each row of ids must hold k distinct
    experts, as a top-k gives (library: lib() by default, or lib_checked())."""
    return _ffn((library or lib()).moe_ffn_decode, "moe_ffn_decode", DECODE, layer, x, ids, w, y, ws, stream)


def forward_decode(layer, x, ids=None, w=None, y=None, ws=None, stream=None):
    """Routing + decode FFN in one call. Returns (y, ids, w)."""
    torch = _torch()
    T = x.shape[0]
    dev = x.device
    if ids is None:
        ids = torch.empty((T, layer.k), dtype=torch.int32, device=dev)
    if w is None:
        w = torch.empty((T, layer.k), dtype=torch.float32, device=dev)
    if y is None:
        y = torch.empty((T, layer.H), dtype=torch.float32, device=dev)
    if ws is None:
        ws = _workspace(workspace_bytes(layer, T, DECODE), dev)
    _dev_check(x, ids, w, y, ws)
    _check(lib().moe_forward_decode(layer.ref, _ptr(x), _x_dtype(x), T, _ptr(ids), _ptr(w), _ptr(y),
                                    _ptr(ws), ws.numel(), _stream(stream)), "moe_forward_decode")
    return y, ids, w


def forward_decode_noalloc(layer, x, ids=None, w=None, y=None, stream=None):
    """moe_forward_decode_noalloc: routing + decode FFN with the library's
    static scratch (no workspace). Returns (y, ids, w)."""
    torch = _torch()
    T = x.shape[0]
    dev = x.device
    if ids is None:
        ids = torch.empty((T, layer.k), dtype=torch.int32, device=dev)
    if w is None:
        w = torch.empty((T, layer.k), dtype=torch.float32, device=dev)
    if y is None:
        y = torch.empty((T, layer.H), dtype=torch.float32, device=dev)
    _dev_check(x, ids, w, y)
    _check(lib().moe_forward_decode_noalloc(layer.ref, _ptr(x), _x_dtype(x), T, _ptr(ids), _ptr(w), _ptr(y),
                                            _stream(stream)), "moe_forward_decode_noalloc")
    return y, ids, w


def ffn_prefill(layer, x, ids, w, y=None, ws=None, stream=None, library=None):
    return _ffn((library or lib()).moe_ffn_prefill, "moe_ffn_prefill", PREFILL, layer, x, ids, w, y, ws, stream)


def dequant_iq2x(blocks, grid, out_dtype=F32, stream=None):
    torch = _torch()
    nb = blocks.numel() // 66
    dt = torch.float32 if out_dtype == F32 else torch.bfloat16
    out = torch.empty(nb * 256, dtype=dt, device=blocks.device)
    _dev_check(blocks, grid)
    _check(lib().moe_dequant_iq2x(_ptr(blocks), _ptr(grid), nb, _ptr(out), out_dtype, _stream(stream)),
           "moe_dequant_iq2x")
    return out


def dequant_q2k(blocks, out_dtype=F32, stream=None):
    torch = _torch()
    nb = blocks.numel() // 84
    dt = torch.float32 if out_dtype == F32 else torch.bfloat16
    out = torch.empty(nb * 256, dtype=dt, device=blocks.device)
    _dev_check(blocks)
    _check(lib().moe_dequant_q2k(_ptr(blocks), nb, _ptr(out), out_dtype, _stream(stream)),
           "moe_dequant_q2k")
    return out


def dequant_mxfp4(blocks, out_dtype=F32, stream=None):
    """Canonical MXFP4 blocks (uint8, 17 bytes each) -> values [n*32]."""
    torch = _torch()
    nb = blocks.numel() // 17
    dt = torch.float32 if out_dtype == F32 else torch.bfloat16
    out = torch.empty(nb * 32, dtype=dt, device=blocks.device)
    _dev_check(blocks)
    _check(lib().moe_dequant_mxfp4(_ptr(blocks), nb, _ptr(out), out_dtype, _stream(stream)), "moe_dequant_mxfp4")
    return out


class ExpertCache:
    """moe_cache_*: the routed experts of `host_layer` (tiled slabs in pinned
    host tensors) served from a pool of `slots` HBM slots.

    host: (gate, up, down) uint8 tensors in pinned host memory, the tiled
    slabs of all E experts; dev_layer: a Layer whose router, grid and shared
    expert are on the device (its routed tensors are not used)."""

    def __init__(self, dev_layer: "Layer", host, slots: int):
        torch = _torch()
        self.host = host
        gate, up, down = host
        for t in host:
            if t.is_cuda or not t.is_pinned():
                raise ValueError("host slabs must be pinned host tensors")
        L = lib()
        nbytes = int(L.moe_cache_pool_bytes(dev_layer.ref, slots))
        if nbytes == 0:
            raise BitMoEError(EINVAL, "moe_cache_pool_bytes")
        self.pool = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
        self.dev_layer = dev_layer
        h = C.c_void_p()
        _check(L.moe_cache_create(dev_layer.ref, _ptr(gate), _ptr(up), _ptr(down), slots, _ptr(self.pool), nbytes,
                                  C.byref(h)), "moe_cache_create")
        self.h = h
        self.slots = slots
        s = LayerStruct()
        _check(L.moe_cache_layer(self.h, C.byref(s)), "moe_cache_layer")
        self.layer = Layer.__new__(Layer)
        self.layer.H, self.layer.I, self.layer.E, self.layer.k = s.H, s.I, s.E, s.k
        self.layer.fmt = s.format
        self.layer.tensors = [self.pool] + list(dev_layer.tensors)
        self.layer.has_shared = dev_layer.has_shared
        self.layer.s = s

    def map(self, ids_host, stream=None):
        """ids_host: int32 host tensor [T, k] -> (slot ids int32 host tensor,
        experts copied)."""
        torch = _torch()
        ids = ids_host.contiguous()
        slot_ids = torch.empty_like(ids)
        loaded = C.c_int(0)
        _check(lib().moe_cache_map(self.h, _ptr(ids), ids.numel(), _ptr(slot_ids), C.byref(loaded),
                                   _stream(stream)), "moe_cache_map")
        return slot_ids, loaded.value

    def stats(self):
        import numpy as np
        hits, misses = C.c_int64(0), C.c_int64(0)
        slots = np.empty(self.slots, dtype=np.int32)
        _check(lib().moe_cache_stats(self.h, C.byref(hits), C.byref(misses), slots.ctypes.data_as(C.c_void_p)),
               "moe_cache_stats")
        return hits.value, misses.value, slots

    def close(self):
        if self.h:
            lib().moe_cache_destroy(self.h)
            self.h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


def quantize_iq2x(w, grid, out=None, stream=None):
    """float32 weights (numel a multiple of 256) -> canonical IQ2X blocks
    uint8 [n, 66] (moe_quantize_iq2x)."""
    torch = _torch()
    nb = w.numel() // 256
    if out is None:
        out = torch.empty((nb, 66), dtype=torch.uint8, device=w.device)
    _dev_check(w, grid, out)
    _check(lib().moe_quantize_iq2x(_ptr(w), _ptr(grid), nb, _ptr(out), _stream(stream)), "moe_quantize_iq2x")
    return out


def quantize_q2k(w, out=None, stream=None):
    """float32 weights (numel a multiple of 256) -> canonical Q2K blocks
    uint8 [n, 84] (moe_quantize_q2k)."""
    torch = _torch()
    nb = w.numel() // 256
    if out is None:
        out = torch.empty((nb, 84), dtype=torch.uint8, device=w.device)
    _dev_check(w, out)
    _check(lib().moe_quantize_q2k(_ptr(w), nb, _ptr(out), _stream(stream)), "moe_quantize_q2k")
    return out


def quantize_mxfp4(w, out=None, stream=None):
    """float32 weights (numel a multiple of 32) -> canonical MXFP4 blocks
    uint8 [n, 17] (moe_quantize_mxfp4)."""
    torch = _torch()
    nb = w.numel() // 32
    if out is None:
        out = torch.empty((nb, 17), dtype=torch.uint8, device=w.device)
    _dev_check(w, out)
    _check(lib().moe_quantize_mxfp4(_ptr(w), nb, _ptr(out), _stream(stream)), "moe_quantize_mxfp4")
    return out


def pack_iq2x(src, E, N, K, stream=None):
    torch = _torch()
    dst = torch.empty_like(src)
    _dev_check(src)
    _check(lib().moe_pack_iq2x(_ptr(src), _ptr(dst), E, N, K, _stream(stream)), "moe_pack_iq2x")
    return dst


def pack_q2k(src, E, N, K, stream=None):
    torch = _torch()
    dst = torch.empty_like(src)
    _dev_check(src)
    _check(lib().moe_pack_q2k(_ptr(src), _ptr(dst), E, N, K, _stream(stream)), "moe_pack_q2k")
    return dst


def pack_mxfp4(src, E, N, K, stream=None):
    torch = _torch()
    dst = torch.empty_like(src)
    _dev_check(src)
    _check(lib().moe_pack_mxfp4(_ptr(src), _ptr(dst), E, N, K, _stream(stream)), "moe_pack_mxfp4")
    return dst


def pack_bf16(src, stream=None):
    torch = _torch()
    N, K = src.shape
    dst = torch.empty_like(src)
    _dev_check(src)
    _check(lib().moe_pack_bf16(_ptr(src), _ptr(dst), N, K, _stream(stream)), "moe_pack_bf16")
    return dst
