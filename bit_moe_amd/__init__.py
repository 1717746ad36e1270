"""bit_moe_amd: the 2-bit (and MXFP4) routed-expert MoE FFN layer on MI355X (gfx950).

Python binding over libbitmoe.so (see include/bitmoe.h).  PyTorch provides
device memory and streams only; every step of the layer runs in the
library's HIP kernels.
"""
from ._lib import (BF16, BitMoEError, DECODE, ExpertCache, F32, FORMAT_2BIT, FORMAT_MXFP4, Layer, PREFILL, SYMBOLS,
                   TIME_DOWN, TIME_GATEUP, bucket, dequant_iq2x, dequant_mxfp4, dequant_q2k, ffn_decode, ffn_prefill,
                   forward_decode, forward_decode_noalloc, lib, lib_checked, quantize_iq2x, quantize_mxfp4, quantize_q2k, pack_bf16, pack_iq2x,
                   pack_mxfp4, pack_q2k, route, route_workspace_bytes, set_timing_events, strerror, topk, version,
                   workspace_bytes)


def layer_from_canonical(H, I, E, k, router_bits, gate, up, down, grid, shared=None, device="cuda",
                         fmt=FORMAT_2BIT):
    """Upload canonical weights (numpy/torch uint8 blocks, bf16 bit arrays) to
    the GPU and convert the quantised and shared tensors to the tiled layout
    with the library's pack entry points.  fmt FORMAT_MXFP4: gate, up and
    down are MXFP4 blocks and grid may be None."""
    import numpy as np
    import torch

    def dev(a, dtype=None):
        t = torch.from_numpy(np.ascontiguousarray(a)) if isinstance(a, np.ndarray) else a
        if dtype is not None:
            t = t.view(dtype)
        return t.to(device).contiguous()

    router = dev(router_bits, torch.bfloat16) if router_bits is not None else \
        torch.zeros((E, H), dtype=torch.bfloat16, device=device)
    if fmt == FORMAT_MXFP4:
        gq = pack_mxfp4(dev(gate).reshape(-1), E, I, H)
        uq = pack_mxfp4(dev(up).reshape(-1), E, I, H)
        dq = pack_mxfp4(dev(down).reshape(-1), E, H, I)
    else:
        gq = pack_iq2x(dev(gate).reshape(-1), E, I, H)
        uq = pack_iq2x(dev(up).reshape(-1), E, I, H)
        dq = pack_q2k(dev(down).reshape(-1), E, H, I)
    g = dev(grid).reshape(-1) if grid is not None else None
    sh = None
    if shared is not None:
        sg, su, sd = (dev(a, torch.bfloat16) for a in shared)
        sh = (pack_bf16(sg), pack_bf16(su), pack_bf16(sd))
    return Layer(H, I, E, k, router, gq, uq, dq, g, sh, fmt=fmt)


__all__ = ["BF16", "BitMoEError", "DECODE", "ExpertCache", "F32", "FORMAT_2BIT", "FORMAT_MXFP4", "Layer", "PREFILL",
           "SYMBOLS", "TIME_DOWN", "TIME_GATEUP", "bucket", "dequant_iq2x", "dequant_mxfp4", "dequant_q2k", "ffn_decode",
           "ffn_prefill", "forward_decode", "forward_decode_noalloc", "layer_from_canonical", "lib_checked", "quantize_iq2x",
           "quantize_mxfp4", "quantize_q2k", "lib", "pack_bf16", "pack_iq2x", "pack_mxfp4", "pack_q2k", "route", "route_workspace_bytes",
           "set_timing_events", "strerror", "topk", "version", "workspace_bytes"]
