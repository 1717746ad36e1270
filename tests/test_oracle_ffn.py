"""Pins of the oracle's MoE FFN (CPU only).

The FFN is the routed SwiGLU expert sum (page "ds4 : analyse pratique pour un
usage documente", section "Support de modeles et choix de quantification":
routed experts quantised, shared expert kept in bf16).  Pins that do not
reuse the oracle's FFN code: dense float64 matrix products against explicitly
dequantised matrices, a closed form on constant blocks, x = 0, linearity in
the routing weights, and equivariance under token and expert relabelling.
"""
import math

import numpy as np
import pytest
import torch

import oracle
import synth

TINY = synth.WORKLOADS["tiny"]


def _dense(layer, e):
    w = layer.w
    G = oracle.dequant_iq2x(layer.gate(e), layer.grid()).reshape(w.I, w.H)
    U = oracle.dequant_iq2x(layer.up(e), layer.grid()).reshape(w.I, w.H)
    D = oracle.dequant_q2k(layer.down(e)).reshape(w.H, w.I)
    return G, U, D


def _x64(x):
    return x.astype(np.float64) if x.dtype == np.float32 else \
        synth.f32_from_bf16_bits(x).astype(np.float64)


def _brute(layer, x, ids, wts):
    xs = _x64(x)
    y = np.zeros((x.shape[0], layer.w.H))
    dense = {}
    for t in range(x.shape[0]):
        for j in range(ids.shape[1]):
            e = int(ids[t, j])
            if e not in dense:
                dense[e] = _dense(layer, e)
            G, U, D = dense[e]
            g, u = G @ xs[t], U @ xs[t]
            h = g / (1 + np.exp(-g)) * u
            y[t] += wts[t, j] * (D @ h)
    if layer.shared() is not None:
        sg, su, sd = (synth.f32_from_bf16_bits(a).astype(np.float64) for a in layer.shared())
        g, u = xs @ sg.T, xs @ su.T
        y += (g / (1 + np.exp(-g)) * u) @ sd.T
    return y


def test_tiny_layer_against_dense_float64_brute_force():
    L = synth.make_layer(TINY)
    x, _ = synth.make_tokens(TINY)
    ids, w = oracle.route(x, L.router(), TINY.k)
    y = oracle.layer_ffn(L, x, ids, w)
    ref = _brute(L, x, ids, w)
    np.testing.assert_allclose(y, ref, rtol=1e-10, atol=1e-12 * np.abs(ref).max())


def test_shared_expert_adds_dense_bf16_ffn():
    wl = TINY.with_(shared=True, seed=7)
    L = synth.make_layer(wl)
    x, _ = synth.make_tokens(wl.with_(x_dtype="bf16"))
    ids, w = oracle.route(x, L.router(), wl.k)
    y = oracle.layer_ffn(L, x, ids, w)
    ref = _brute(L, x, ids, w)
    np.testing.assert_allclose(y, ref, rtol=1e-10, atol=1e-12 * np.abs(ref).max())


def test_single_expert_weight_one_is_textbook_dense_ffn():
    """k = 1 with weight 1 equals torch's SwiGLU FFN of that expert's
    explicitly dequantised matrices."""
    L = synth.make_layer(TINY)
    x, _ = synth.make_tokens(TINY)
    e = 5
    ids = np.full((TINY.T, 1), e, dtype=np.int32)
    w = np.ones((TINY.T, 1))
    y = oracle.moe_ffn(TINY.H, TINY.I, TINY.E, 1, L.grid(), {e: L.gate(e)}, {e: L.up(e)},
                       {e: L.down(e)}, None, x, ids, w)
    G, U, D = (torch.from_numpy(m) for m in _dense(L, e))
    xt = torch.from_numpy(x.astype(np.float64))
    ref = (torch.nn.functional.silu(xt @ G.T) * (xt @ U.T)) @ D.T
    np.testing.assert_allclose(y, ref.numpy(), rtol=1e-10, atol=1e-12 * float(ref.abs().max()))


def test_zero_activation_gives_zero_output():
    L = synth.make_layer(TINY)
    x = np.zeros((3, TINY.H), dtype=np.float32)
    ids, w = oracle.route(x, L.router(), TINY.k)
    y = oracle.layer_ffn(L, x, ids, w)
    assert np.all(y == 0.0)


def _const_iq2x(n_blocks, d_bits, grp_bytes):
    b = np.zeros((n_blocks, 66), dtype=np.uint8)
    b[:, 0] = d_bits & 0xFF
    b[:, 1] = d_bits >> 8
    b[:, 2:] = np.tile(np.frombuffer(bytes(grp_bytes), dtype=np.uint8), 8)
    return b


def test_closed_form_constant_blocks():
    """Every gate weight a, every up weight b, every down weight c, x = 1:
    g = H*a, u = H*b, h = silu(H*a)*H*b, y = w * I * c * h."""
    H, I = 256, 256
    grid = np.ones((256, 8), dtype=np.uint8)               # all magnitudes 1
    # gate: d = 1.0, s = 0 -> a = 0.125; up: d = 0.5, s = 1 -> b = 0.5*1.5/4 = 0.1875
    gate = _const_iq2x(I, 0x3C00, [0, 0, 0, 0, 0, 0, 0, 0])
    up = _const_iq2x(I, 0x3800, [0, 0, 0, 0, 0, 0, 0, 0x10])
    # down: d = 0.25, scale 2, q = 1, min 0 -> c = 0.5
    down = np.zeros((H, 84), dtype=np.uint8)
    down[:, :16] = 0x02
    down[:, 16:80] = 0x55                                    # every 2-bit quant = 1
    down[:, 80:82] = np.array([0.25], dtype=np.float16).view(np.uint8)
    x = np.ones((2, H), dtype=np.float32)
    ids = np.array([[0], [0]], dtype=np.int32)
    w = np.array([[1.0], [0.375]])
    y = oracle.moe_ffn(H, I, 1, 1, grid, [gate], [up], [down], None, x, ids, w)
    a, b, c = 0.125, 0.1875, 0.5
    g, u = H * a, H * b
    h = g / (1 + math.exp(-g)) * u
    for t in range(2):
        np.testing.assert_allclose(y[t], w[t, 0] * I * c * h, rtol=1e-14)


def test_linear_in_routing_weights():
    L = synth.make_layer(TINY)
    x, _ = synth.make_tokens(TINY)
    ids, w = oracle.route(x, L.router(), TINY.k)
    y1 = oracle.layer_ffn(L, x, ids, w)
    y2 = oracle.layer_ffn(L, x, ids, 3.0 * w)
    np.testing.assert_allclose(y2, 3.0 * y1, rtol=1e-13, atol=1e-15)
    # slot contributions add: weight (w0, 0) + (0, w1) == (w0, w1)
    wa, wb = w.copy(), w.copy()
    wa[:, 1] = 0
    wb[:, 0] = 0
    ya = oracle.layer_ffn(L, x, ids, wa)
    yb = oracle.layer_ffn(L, x, ids, wb)
    np.testing.assert_allclose(ya + yb, y1, rtol=1e-12, atol=1e-14)


def test_token_permutation_equivariance():
    L = synth.make_layer(TINY)
    x, _ = synth.make_tokens(TINY)
    ids, w = oracle.route(x, L.router(), TINY.k)
    y = oracle.layer_ffn(L, x, ids, w)
    p = np.array([2, 0, 3, 1])
    yp = oracle.layer_ffn(L, x[p], ids[p], w[p])
    np.testing.assert_array_equal(yp, y[p])


def test_expert_relabelling_invariance():
    """Permuting the router rows and the expert slabs together leaves y unchanged."""
    L = synth.make_layer(TINY)
    x, _ = synth.make_tokens(TINY)
    perm = np.array([3, 7, 0, 5, 1, 6, 2, 4])                # new expert i = old perm[i]
    wr = L.router()
    ids, w = oracle.route(x, wr, TINY.k)
    y = oracle.layer_ffn(L, x, ids, w)
    wr2 = wr[perm]
    ids2, w2 = oracle.route(x, wr2, TINY.k)
    inv = np.argsort(perm)
    np.testing.assert_array_equal(ids2, inv[ids])
    g = {i: L.gate(int(perm[i])) for i in range(TINY.E)}
    u = {i: L.up(int(perm[i])) for i in range(TINY.E)}
    d = {i: L.down(int(perm[i])) for i in range(TINY.E)}
    y2 = oracle.moe_ffn(TINY.H, TINY.I, TINY.E, TINY.k, L.grid(), g, u, d, None, x, ids2, w2)
    np.testing.assert_array_equal(y2, y)


@pytest.mark.parametrize("name", ["tiny"])
def test_margin_predicate_keeps_ids_stable_under_fp32(name):
    """With the margin predicate, fp32 logits (any summation order) select
    the same experts as fp64 logits."""
    wl = synth.WORKLOADS[name]
    L = synth.make_layer(wl)
    wr = L.router()
    x, att = synth.make_tokens(wl, accept=lambda t, r: oracle.margin_ok(r, wr, wl.k, 1e-3))
    ids, _ = oracle.route(x, wr, wl.k)
    l32 = (x.astype(np.float32) @ synth.f32_from_bf16_bits(wr).T).astype(np.float64)
    ids32, _ = oracle.topk(l32, wl.k)
    np.testing.assert_array_equal(ids32, ids)
