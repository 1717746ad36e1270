"""CPU oracle for the 2-bit routed-expert MoE layer (ctypes over oracle.c).

TEST INFRASTRUCTURE ONLY: imported by ``tests/``, by the smoke check and by
the CPU-baseline leg of ``bench.py``; never by the library.  Every function is
the plain definition evaluated in double precision (see oracle.c for the
sources and readings).

Parity status: dequantisation, routing, bucketing and the FFN are pinned by
tests that do not re-use this code (hand-decoded golden blocks, closed forms,
invariants, and dense float64 matrix products on small shapes); the
quantizer (quant.c) by exact round trips of representable blocks, brute-force
optimality of every run and sub-block choice, and never-worse-than-start.
"""
from __future__ import annotations

import ctypes as C
import os

import numpy as np

from . import build as _build

_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_build.LIB):
            _build.build()
        L = C.CDLL(_build.LIB)
        P, I64, I32 = C.c_void_p, C.c_int64, C.c_int
        L.oracle_fp16_to_double.argtypes = [C.c_uint16]
        L.oracle_fp16_to_double.restype = C.c_double
        L.oracle_bf16_to_double.argtypes = [C.c_uint16]
        L.oracle_bf16_to_double.restype = C.c_double
        L.oracle_dequant_iq2x.argtypes = [P, P, I64, P]
        L.oracle_dequant_q2k.argtypes = [P, I64, P]
        L.oracle_router_logits.argtypes = [P, I32, I32, I32, P, I32, P]
        L.oracle_topk.argtypes = [P, I32, I32, I32, P, P]
        L.oracle_bucket.argtypes = [P, I32, I32, I32, P, P, P]
        L.oracle_moe_ffn.argtypes = [I32, I32, I32, I32, P, P, P, P, P, P, P,
                                     P, I32, I32, P, P, P]
        L.oracle_moe_ffn_mxfp4.argtypes = [I32, I32, I32, I32, P, P, P, P, P, P,
                                           P, I32, I32, P, P, P]
        L.oracle_dequant_mxfp4.argtypes = [P, I64, P]
        L.oracle_quantize_iq2x.argtypes = [P, P, I64, P]
        L.oracle_quantize_q2k.argtypes = [P, I64, P]
        L.oracle_quantize_mxfp4.argtypes = [P, I64, P]
        L.oracle_max_threads.restype = I32
        L.oracle_set_threads.argtypes = [I32]
        _lib = L
    return _lib


def _p(a: np.ndarray):
    return a.ctypes.data_as(C.c_void_p)


def set_threads(n: int) -> None:
    lib().oracle_set_threads(int(n))


def max_threads() -> int:
    return int(lib().oracle_max_threads())


def fp16_to_double(h: int) -> float:
    return float(lib().oracle_fp16_to_double(int(h)))


def dequant_iq2x(blocks: np.ndarray, grid: np.ndarray) -> np.ndarray:
    """Canonical IQ2X blocks uint8 [n, 66] -> float64 [n * 256] (exact)."""
    b = np.ascontiguousarray(blocks, dtype=np.uint8).reshape(-1, 66)
    g = np.ascontiguousarray(grid, dtype=np.uint8).reshape(256, 8)
    out = np.empty(b.shape[0] * 256, dtype=np.float64)
    lib().oracle_dequant_iq2x(_p(b), _p(g), b.shape[0], _p(out))
    return out


def dequant_q2k(blocks: np.ndarray) -> np.ndarray:
    """Canonical Q2K blocks uint8 [n, 84] -> float64 [n * 256] (exact)."""
    b = np.ascontiguousarray(blocks, dtype=np.uint8).reshape(-1, 84)
    out = np.empty(b.shape[0] * 256, dtype=np.float64)
    lib().oracle_dequant_q2k(_p(b), b.shape[0], _p(out))
    return out


def quantize_iq2x(w: np.ndarray, grid: np.ndarray) -> np.ndarray:
    """float32 weights [n * 256] -> canonical IQ2X blocks uint8 [n, 66]
    (error-minimising search of quant.c)."""
    wf = np.ascontiguousarray(w, dtype=np.float32).reshape(-1)
    assert wf.size % 256 == 0
    g = np.ascontiguousarray(grid, dtype=np.uint8).reshape(256, 8)
    out = np.empty((wf.size // 256, 66), dtype=np.uint8)
    lib().oracle_quantize_iq2x(_p(wf), _p(g), out.shape[0], _p(out))
    return out


def quantize_mxfp4(w: np.ndarray) -> np.ndarray:
    """float32 weights [n * 32] -> canonical MXFP4 blocks uint8 [n, 17]
    (OCP shared exponent with the two-way scale search of quant.c)."""
    wf = np.ascontiguousarray(w, dtype=np.float32).reshape(-1)
    assert wf.size % 32 == 0
    out = np.empty((wf.size // 32, 17), dtype=np.uint8)
    lib().oracle_quantize_mxfp4(_p(wf), out.shape[0], _p(out))
    return out


def quantize_q2k(w: np.ndarray) -> np.ndarray:
    """float32 weights [n * 256] -> canonical Q2K blocks uint8 [n, 84]."""
    wf = np.ascontiguousarray(w, dtype=np.float32).reshape(-1)
    assert wf.size % 256 == 0
    out = np.empty((wf.size // 256, 84), dtype=np.uint8)
    lib().oracle_quantize_q2k(_p(wf), out.shape[0], _p(out))
    return out


def dequant_mxfp4(blocks: np.ndarray) -> np.ndarray:
    """Canonical MXFP4 blocks uint8 [n, 17] -> float64 [n * 32] (exact)."""
    b = np.ascontiguousarray(blocks, dtype=np.uint8).reshape(-1, 17)
    out = np.empty(b.shape[0] * 32, dtype=np.float64)
    lib().oracle_dequant_mxfp4(_p(b), b.shape[0], _p(out))
    return out


def _x_args(x: np.ndarray):
    if x.dtype == np.float32:
        return np.ascontiguousarray(x), 0
    if x.dtype == np.uint16:
        return np.ascontiguousarray(x), 1
    raise TypeError("x must be float32 or uint16 (bf16 bits)")


def router_logits(x: np.ndarray, wr_bits: np.ndarray) -> np.ndarray:
    """x [T,H] (float32 or bf16 bits), router bf16 bits [E,H] -> float64 [T,E]."""
    xc, dt = _x_args(x)
    T, H = xc.shape
    wr = np.ascontiguousarray(wr_bits, dtype=np.uint16)
    E = wr.shape[0]
    out = np.empty((T, E), dtype=np.float64)
    lib().oracle_router_logits(_p(xc), dt, T, H, _p(wr), E, _p(out))
    return out


def topk(logits: np.ndarray, k: int):
    """float64 (or float32, widened exactly) [T,E] -> ids int32 [T,k], w float64 [T,k]."""
    l = np.ascontiguousarray(logits, dtype=np.float64)
    T, E = l.shape
    ids = np.empty((T, k), dtype=np.int32)
    w = np.empty((T, k), dtype=np.float64)
    lib().oracle_topk(_p(l), T, E, k, _p(ids), _p(w))
    return ids, w


def route(x: np.ndarray, wr_bits: np.ndarray, k: int):
    return topk(router_logits(x, wr_bits), k)


def bucket(ids: np.ndarray, E: int):
    """ids int32 [T,k] -> counts [E], offsets [E+1], perm [T*k] (int32)."""
    i = np.ascontiguousarray(ids, dtype=np.int32)
    T, k = i.shape
    counts = np.empty(E, dtype=np.int32)
    offsets = np.empty(E + 1, dtype=np.int32)
    perm = np.empty(T * k, dtype=np.int32)
    lib().oracle_bucket(_p(i), T, k, E, _p(counts), _p(offsets), _p(perm))
    return counts, offsets, perm


def moe_ffn(H, I, E, k, grid, gate, up, down, shared, x, ids, w, fmt: str = "2bit") -> np.ndarray:
    """Routed (+ shared) SwiGLU FFN in float64.

    fmt "2bit": gate/up IQ2X, down Q2K (grid: the codebook); "mxfp4": all
    three MXFP4 (grid unused).

    gate/up/down: mappings expert -> canonical block array of that expert
    (any expert referenced by ``ids`` must be present).  shared: None or
    (gate [I,H], up [I,H], down [H,I]) bf16 bits.  Returns y float64 [T,H].
    """
    xc, dt = _x_args(x)
    T = xc.shape[0]
    assert xc.shape[1] == H
    ids_c = np.ascontiguousarray(ids, dtype=np.int32).reshape(T, k)
    w_c = np.ascontiguousarray(w, dtype=np.float64).reshape(T, k)
    keep = []

    def ptrs(src, nbytes):
        arr = (C.c_void_p * E)()
        for e in range(E):
            blk = src.get(e) if isinstance(src, dict) else (src[e] if e < len(src) else None)
            if blk is None:
                continue
            b = np.ascontiguousarray(blk, dtype=np.uint8)
            assert b.size == nbytes, (e, b.size, nbytes)
            keep.append(b)
            arr[e] = b.ctypes.data
        return arr

    used = set(int(e) for e in ids_c.ravel())
    for e in used:
        for src in (gate, up, down):
            has = (e in src) if isinstance(src, dict) else (e < len(src))
            if not has:
                raise KeyError(f"expert {e} missing")
    if fmt == "mxfp4":
        g_p = ptrs(gate, I * (H // 32) * 17)
        u_p = ptrs(up, I * (H // 32) * 17)
        d_p = ptrs(down, H * (I // 32) * 17)
    else:
        g_p = ptrs(gate, I * (H // 256) * 66)
        u_p = ptrs(up, I * (H // 256) * 66)
        d_p = ptrs(down, H * (I // 256) * 84)
    if shared is not None:
        sg, su, sd = (np.ascontiguousarray(a, dtype=np.uint16) for a in shared)
        assert sg.shape == (I, H) and su.shape == (I, H) and sd.shape == (H, I)
        keep += [sg, su, sd]
        sgp, sup, sdp = _p(sg), _p(su), _p(sd)
    else:
        sgp = sup = sdp = None
    y = np.empty((T, H), dtype=np.float64)
    if fmt == "mxfp4":
        lib().oracle_moe_ffn_mxfp4(H, I, E, k, g_p, u_p, d_p, sgp, sup, sdp,
                                   _p(xc), dt, T, _p(ids_c), _p(w_c), _p(y))
        return y
    gr = np.ascontiguousarray(grid, dtype=np.uint8).reshape(256, 8)
    lib().oracle_moe_ffn(H, I, E, k, _p(gr), g_p, u_p, d_p, sgp, sup, sdp,
                         _p(xc), dt, T, _p(ids_c), _p(w_c), _p(y))
    return y


def layer_ffn(layer, x, ids, w, experts=None) -> np.ndarray:
    """Convenience: FFN over a synth.Layer, generating only the experts used."""
    wl = layer.w
    used = sorted(set(int(e) for e in np.asarray(ids).ravel())) if experts is None else experts
    gate = {e: layer.gate(e) for e in used}
    up = {e: layer.up(e) for e in used}
    down = {e: layer.down(e) for e in used}
    return moe_ffn(wl.H, wl.I, wl.E, wl.k, layer.grid(), gate, up, down,
                   layer.shared(), x, ids, w, fmt=getattr(wl, "fmt", "2bit"))


def margin_ok(x_row: np.ndarray, wr_bits: np.ndarray, k: int, margin: float) -> bool:
    """True when the k+1 largest router logits of one token are separated by
    at least ``margin`` (so accumulation order cannot change the top-k)."""
    l = np.sort(router_logits(x_row.reshape(1, -1), wr_bits)[0])[::-1]
    gaps = l[:k] - l[1:k + 1]
    return bool(np.all(gaps >= margin))
