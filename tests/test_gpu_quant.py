"""GPU parity: the quantizer (moe_quantize_iq2x / moe_quantize_q2k) against
the oracle's encoder, byte for byte: every choice is a decision taken in
double precision in a fixed order on both sides, so the blocks must be
identical.  Inputs: Gaussian weights at the tiny config's shapes and scales,
weights spanning many binades, blocks whose values the formats represent
exactly (the search must find zero error), edge cases (zeros, negative zero,
constants, one sign), and sampled superblocks of a full-size expert tensor
(2048 x 7168) encoded in one launch."""
import numpy as np
import pytest

import oracle
import synth
from _gpu import require_gpu, say, torch

pytestmark = pytest.mark.gpu

GRID = synth.make_layer(synth.WORKLOADS["tiny"]).grid()


def _gpu(fmt, w):
    import bit_moe_amd as bm
    wd = torch.from_numpy(np.ascontiguousarray(w, dtype=np.float32)).cuda()
    if fmt == "iq2x":
        out = bm.quantize_iq2x(wd, torch.from_numpy(GRID).cuda())
    else:
        out = bm.quantize_q2k(wd)
    torch.cuda.synchronize()
    return out.cpu().numpy()


def _oracle(fmt, w):
    return oracle.quantize_iq2x(w, GRID) if fmt == "iq2x" else oracle.quantize_q2k(w)


def _same(fmt, w, what):
    g, o = _gpu(fmt, w), _oracle(fmt, w)
    bad = np.nonzero((g != o).any(axis=1))[0]
    say(f"[quant] {fmt} {what}: {g.shape[0]} superblocks, {len(bad)} differ")
    np.testing.assert_array_equal(g, o)


@pytest.mark.parametrize("fmt", ["iq2x", "q2k"])
def test_gaussian_weights_at_the_tiny_shapes(fmt):
    """The tiny config's gate/up (512 x 256) and down (256 x 512) tensors,
    8 experts, as N(0, 0.02) weights."""
    require_gpu()
    rng = np.random.default_rng(21)
    w = (rng.standard_normal(8 * 512 * 256) * 0.02).astype(np.float32)
    _same(fmt, w, "tiny-shaped N(0, 0.02)")


@pytest.mark.parametrize("fmt", ["iq2x", "q2k"])
def test_weights_over_many_binades_and_edge_cases(fmt):
    require_gpu()
    rng = np.random.default_rng(22)
    w = (rng.standard_normal(256 * 96) * np.exp2(rng.integers(-30, 10, 256 * 96))).astype(np.float32)
    blocks = w.reshape(-1, 256)
    blocks[0] = 0.0                                   # all zero
    blocks[1] = -0.0                                  # negative zero
    blocks[2] = 0.125                                 # constant
    blocks[3] = np.abs(blocks[3])                     # one sign
    blocks[4] = -np.abs(blocks[4])
    blocks[5, :] = 0.0
    blocks[5, 77] = 3.0                               # one nonzero weight
    blocks[6] *= 1e-6                                 # scales in fp16's subnormal range
    blocks[7] = np.where(np.arange(256) % 2, 1e-3, -1e-3)
    _same(fmt, blocks.reshape(-1), "binades + edge cases")


def test_representable_blocks_come_back_exactly():
    """Weights decoded from blocks built so the encoder's scales equal the
    blocks' own: zero error is reachable, and both encoders reach it."""
    require_gpu()
    import test_oracle_quant as tq
    rng = np.random.default_rng(23)
    bi = tq._iq2x_representable(rng, 32)
    wi = oracle.dequant_iq2x(bi, GRID).astype(np.float32)
    _same("iq2x", wi, "representable")
    np.testing.assert_array_equal(oracle.dequant_iq2x(_gpu("iq2x", wi), GRID), wi)
    bq = tq._q2k_representable(rng, 32)
    wq = oracle.dequant_q2k(bq).astype(np.float32)
    _same("q2k", wq, "representable")
    np.testing.assert_array_equal(oracle.dequant_q2k(_gpu("q2k", wq)), wq)


@pytest.mark.parametrize("fmt", ["iq2x", "q2k"])
def test_full_size_expert_tensor_sampled(fmt):
    """A 2048 x 7168 tensor (57344 superblocks) encoded in one launch; the
    oracle checks 1024 sampled superblocks, the first and last included."""
    require_gpu()
    rng = np.random.default_rng(24)
    n = 2048 * 7168 // 256
    w = (rng.standard_normal(n * 256) / (10.6 * np.sqrt(7168))).astype(np.float32)
    g = _gpu(fmt, w)
    rows = np.unique(np.concatenate([[0, n - 1], rng.choice(n, 1022, replace=False)]))
    o = _oracle(fmt, w.reshape(n, 256)[rows].reshape(-1))
    say(f"[quant] {fmt} full tensor: {len(rows)} sampled superblocks")
    np.testing.assert_array_equal(g[rows], o)


def test_mxfp4_quantizer_matches_oracle():
    """moe_quantize_mxfp4 against the oracle's encoder, byte for byte:
    Gaussian weights over many binades, fp32 subnormals and values near the
    top of fp32's range, ties at every E2M1 midpoint, zero, negative zero and
    constant blocks, and a full 2048 x 7168 expert tensor in one launch."""
    require_gpu()
    import bit_moe_amd as bm
    rng = np.random.default_rng(31)
    w = (rng.standard_normal(32 * 4096) * np.exp2(rng.integers(-60, 60, 32 * 4096))).astype(np.float32)
    b = w.reshape(-1, 32)
    b[0] = 0.0
    b[1] = -0.0
    b[2] = 0.37
    b[3] = -1e-40                                               # fp32 subnormals
    b[4] = rng.standard_normal(32).astype(np.float32) * np.float32(1e-42)
    b[5] = rng.standard_normal(32).astype(np.float32) * np.float32(1e37)
    b[6, :8] = [6.0, 0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0]     # ties at scale 1
    b[6, 8:] = 0.5
    full = (rng.standard_normal(2048 * 7168) * 0.02).astype(np.float32)
    for what, x in (("edge blocks over many binades", w), ("one 2048 x 7168 tensor", full)):
        g = bm.quantize_mxfp4(torch.from_numpy(x).cuda())
        torch.cuda.synchronize()
        g = g.cpu().numpy()
        o = oracle.quantize_mxfp4(x)
        say(f"[quant] mxfp4 {what}: {g.shape[0]} blocks, {int((g != o).any(axis=1).sum())} differ")
        np.testing.assert_array_equal(g, o)
