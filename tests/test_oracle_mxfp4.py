"""Pins of the oracle's MXFP4 path (CPU only): the pages' MXFP4 variant
keeps DeepSeek's released FP4 expert weights ("ds4 : analyse pratique pour
un usage documente", section "Support de modeles et choix de
quantification").  The element and scale encodings are the OCP MX ones
(E2M1, E8M0) in GGML's block byte order.

 - hand-decoded blocks with hand-computed values (tests/golden/mxfp4_hand.json);
 - an independent numpy decoder, bit-equal on random blocks;
 - the FFN against dense float64 products of explicitly decoded weights.
"""
import json
import os

import numpy as np
import pytest

import oracle
import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "mxfp4_hand.json")


@pytest.mark.parametrize("case", [c["name"] for c in json.load(open(GOLDEN))["cases"]])
def test_mxfp4_golden(case):
    c = next(c for c in json.load(open(GOLDEN))["cases"] if c["name"] == case)
    blk = np.frombuffer(bytes.fromhex(c["hex"]), dtype=np.uint8)
    assert blk.size == 17
    got = oracle.dequant_mxfp4(blk)
    exp = np.array(c["expect"], dtype=np.float64)
    np.testing.assert_array_equal(got, exp)
    np.testing.assert_array_equal(np.signbit(got), np.signbit(exp))     # -0 stays -0


_E2M1 = np.array([0, 0.5, 1, 1.5, 2, 3, 4, 6], dtype=np.float64)


def _np_mxfp4(blocks):
    b = np.ascontiguousarray(blocks, dtype=np.uint8).reshape(-1, 17)
    codes = np.concatenate([b[:, 1:] & 0xF, b[:, 1:] >> 4], axis=1)          # [n, 32]: j, then j + 16
    mag = _E2M1[codes & 7]
    v = np.where(codes & 8, -mag, mag)
    with np.errstate(invalid="ignore"):
        scale = np.where(b[:, 0] == 255, np.nan, np.ldexp(1.0, b[:, 0].astype(np.int64) - 127))
        return (v * scale[:, None]).reshape(-1)


def test_numpy_decoder_agrees_on_random_blocks():
    rng = np.random.default_rng(31)
    blk = rng.integers(0, 256, size=(1 << 16, 17), dtype=np.uint8)
    a, b = _np_mxfp4(blk), oracle.dequant_mxfp4(blk)
    np.testing.assert_array_equal(a, b)
    f = np.isfinite(a)
    np.testing.assert_array_equal(a[f].view(np.uint64), b[f].view(np.uint64))
    assert np.isnan(b[np.repeat(blk[:, 0] == 255, 32)]).all()


def test_ffn_matches_dense_float64_products():
    """Tiny MXFP4 layer with a shared expert: the oracle FFN against numpy
    dense matrix products of the decoded weights."""
    w = synth.WORKLOADS["tiny"].with_(name="tiny_mx", fmt="mxfp4", shared=True, seed=33)
    L = synth.make_layer(w)
    x, _ = synth.make_tokens(w)
    ids, rw = oracle.route(x, L.router(), w.k)
    y = oracle.layer_ffn(L, x, ids, rw)
    xd = x.astype(np.float64)
    ref = np.zeros((w.T, w.H))
    for t in range(w.T):
        for j in range(w.k):
            e = ids[t, j]
            G = _np_mxfp4(L.gate(e)).reshape(w.I, w.H)
            U = _np_mxfp4(L.up(e)).reshape(w.I, w.H)
            D = _np_mxfp4(L.down(e)).reshape(w.H, w.I)
            g, u = G @ xd[t], U @ xd[t]
            ref[t] += rw[t, j] * (D @ (g / (1 + np.exp(-g)) * u))
        sg, su, sd = (synth.f32_from_bf16_bits(a).astype(np.float64) for a in L.shared())
        g, u = sg @ xd[t], su @ xd[t]
        ref[t] += sd @ (g / (1 + np.exp(-g)) * u)
    np.testing.assert_allclose(y, ref, rtol=1e-10, atol=1e-12 * np.abs(ref).max())
