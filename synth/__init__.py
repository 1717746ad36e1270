"""Seeded synthetic inputs for the 2-bit routed-expert MoE layer.

This package only draws bytes and numbers; it performs none of the layer's
arithmetic (no routing, no dequantisation, no products).  Both the CPU oracle
(in ``oracle/``) and the HIP library consume exactly the bytes it produces.
"""
from .gen import (WORKLOADS, Workload, Layer, make_layer, make_tokens,
                  zipf_logits, bf16_bits_from_f32, f32_from_bf16_bits,
                  IQ2X_BLOCK_BYTES, Q2K_BLOCK_BYTES, MXFP4_BLOCK_BYTES, QK)

__all__ = ["WORKLOADS", "Workload", "Layer", "make_layer", "make_tokens",
           "zipf_logits", "bf16_bits_from_f32", "f32_from_bf16_bits",
           "IQ2X_BLOCK_BYTES", "Q2K_BLOCK_BYTES", "MXFP4_BLOCK_BYTES", "QK"]
