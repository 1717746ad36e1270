"""GPU parity of the MXFP4 routed-expert variant (OCP Microscaling FP4:
E2M1 elements, one E8M0 scale per 32 weights, GGML's block order).

 - Standalone dequantisation, bit-exact: every value element * 2^(X-127)
   is exact in float64, so the fp32 output must equal float32(oracle) bit
   for bit (+-inf past fp32's range, NaN for X = 255) and the bf16 output
   its round-to-nearest-even; all 256 scale bytes and all 16 element codes
   are covered.  The kernel uses the hardware conversion that the FFN
   kernels use, so this also pins that conversion.
 - The pack layout, against the header's description written out in numpy.
 - The FFN (decode and prefill entry points, and the fused decode with its
   own routing) against the oracle, max|err| <= 2e-2 * rms(oracle output).
"""
import numpy as np
import pytest

import oracle
import synth
from _gpu import (W_TOL, assert_close_rms, device_layer, require_gpu, say, synth_layer, torch, x_to_device)
from test_gpu_ffn import _oracle_rows, _routing, _sample_rows

pytestmark = pytest.mark.gpu


def _mx(name):
    w = synth.WORKLOADS[name]
    return w.with_(name=f"{w.name}_mxfp4", fmt="mxfp4")


def _gpu_dequant(blocks, out_dtype):
    import bit_moe_amd as bm
    b = torch.from_numpy(np.ascontiguousarray(blocks).reshape(-1)).cuda()
    out = bm.dequant_mxfp4(b, out_dtype)
    torch.cuda.synchronize()
    return out


def _expect(ref64):
    with np.errstate(over="ignore", invalid="ignore"):
        return ref64.astype(np.float32)


@pytest.mark.parametrize("out_dtype", [0, 1])
def test_dequant_every_scale_and_code(out_dtype):
    require_gpu()
    rng = np.random.default_rng(61)
    per = 8
    blk = rng.integers(0, 256, size=(256 * per, 17), dtype=np.uint8)
    blk[:, 0] = np.repeat(np.arange(256, dtype=np.uint8), per)
    # every element code in both nibbles of every scale's blocks
    codes = np.arange(16, dtype=np.uint8)
    blk[::per, 1:17] = codes | (codes[::-1] << 4)
    ref = oracle.dequant_mxfp4(blk)
    nan = np.isnan(ref)
    assert nan.sum() == per * 32
    out = _gpu_dequant(blk, out_dtype)
    if out_dtype == 0:
        got = out.cpu().numpy()
        np.testing.assert_array_equal(got[~nan].view(np.uint32), _expect(ref[~nan]).view(np.uint32))
        assert np.all(np.isnan(got[nan]))
    else:
        got = out.view(torch.int16).cpu().numpy().view(np.uint16)
        np.testing.assert_array_equal(got[~nan], synth.bf16_bits_from_f32(_expect(ref[~nan])))
        assert np.all(((got[nan] & 0x7F80) == 0x7F80) & ((got[nan] & 0x7F) != 0))
    say(f"[mxfp4] dequant dtype={out_dtype}: {len(ref)} values bit-exact, {nan.sum()} NaN")


def test_dequant_layer_tensors_and_empty():
    require_gpu()
    w = _mx("tiny")
    L = synth_layer(w)
    for e in (0, 7):
        for blk in (L.gate(e), L.up(e), L.down(e)):
            np.testing.assert_array_equal(_gpu_dequant(blk, 0).cpu().numpy().view(np.uint32),
                                          _expect(oracle.dequant_mxfp4(blk)).view(np.uint32))
    assert _gpu_dequant(np.zeros((0, 17), np.uint8), 0).numel() == 0


def _tiled_mxfp4_numpy(canon, N, K):
    """The header's tiled MXFP4 slab: pieces ((P nb + kb) 8 + c) 64 + r of
    16 bytes (byte i = weight 2i | weight 2i+1 << 4), then the scale bytes
    ((P nb + kb) 64 + r) 8 + c."""
    nb = K // 256
    b = canon.reshape(N, nb, 8, 17)
    qs = b[..., 1:17]
    j = np.arange(32)
    el = np.where(j < 16, qs[..., j % 16] & 15, qs[..., j % 16] >> 4)        # [N][nb][8][32] codes
    pairs = (el[..., 0::2] | (el[..., 1::2] << 4)).astype(np.uint8)         # [N][nb][8][16]
    pieces = pairs.reshape(N // 64, 64, nb, 8, 16).transpose(0, 2, 3, 1, 4)  # [P][kb][c][r][16]
    scales = b[..., 0].reshape(N // 64, 64, nb, 8).transpose(0, 2, 1, 3)     # [P][kb][r][c]
    return np.concatenate([pieces.reshape(-1), scales.reshape(-1)])


def test_pack_mxfp4_matches_documented_layout():
    require_gpu()
    import bit_moe_amd as bm
    w = _mx("tiny")
    L = synth_layer(w)
    for e in (0, 5):
        for blk, N, K in ((L.gate(e), w.I, w.H), (L.down(e), w.H, w.I)):
            got = bm.pack_mxfp4(torch.from_numpy(blk.reshape(-1)).cuda(), 1, N, K).cpu().numpy()
            np.testing.assert_array_equal(got, _tiled_mxfp4_numpy(blk, N, K))


@pytest.mark.parametrize("mode", ["decode", "prefill"])
def test_tiny_all_tokens(mode):
    require_gpu()
    from test_gpu_ffn import _gpu_ffn
    w = _mx("tiny")
    x, _ = synth.make_tokens(w)
    ids, wt = _routing(w, x)
    ref = _oracle_rows(w, x, ids, wt, np.arange(w.T))
    assert_close_rms(_gpu_ffn(w, x, ids, wt, mode), ref, what=f"mxfp4 tiny/{mode}")


@pytest.mark.parametrize("mode", ["decode", "prefill"])
def test_tiny_shared_ragged_both_dtypes(mode):
    require_gpu()
    from test_gpu_ffn import _gpu_ffn
    for xd, T in (("bf16", 37), ("f32", 5)):
        w = _mx("tiny").with_(name=f"tiny_mx_sh_{xd}", T=T, shared=True, x_dtype=xd, seed=23)
        x, _ = synth.make_tokens(w)
        ids, wt = _routing(w, x)
        ref = _oracle_rows(w, x, ids, wt, np.arange(T))
        assert_close_rms(_gpu_ffn(w, x, ids, wt, mode), ref, what=f"mxfp4 tiny-shared/{xd}/{mode}/T={T}")


@pytest.mark.parametrize("T", [1, 2, 3, 8, 16, 64, 200])
def test_tiny_decode_batch_paths(T):
    """T = 1: one expert per workgroup item; 2 to 8: experts chosen by one
    and by several tokens in the same launches (passes of up to 4 tokens);
    16 and 64: experts chosen by several tokens on the prefill kernels
    beside the single-token ones; 200: the several-token decode passes (four
    tokens per pass)."""
    require_gpu()
    from test_gpu_ffn import _gpu_ffn
    w = _mx("tiny").with_(name=f"tiny_mx_b{T}", T=T, x_dtype="bf16", shared=True, seed=40 + T)
    x, _ = synth.make_tokens(w)
    ids, wt = _routing(w, x)
    ref = _oracle_rows(w, x, ids, wt, np.arange(T))
    assert_close_rms(_gpu_ffn(w, x, ids, wt, "decode"), ref, what=f"mxfp4 tiny decode T={T}")


@pytest.mark.parametrize("name", ["decode_b1", "decode_b16_zipf"])
def test_decode_full_size(name):
    require_gpu()
    from test_gpu_ffn import _gpu_ffn
    w = _mx(name)
    x, _ = synth.make_tokens(w)
    ids, wt = _routing(w, x)
    ref = _oracle_rows(w, x, ids, wt, np.arange(w.T))
    assert_close_rms(_gpu_ffn(w, x, ids, wt, "decode"), ref, what=f"mxfp4 {name}")


@pytest.mark.parametrize("name", ["prefill_2k", "prefill_8k_zipf"])
def test_prefill_full_size_sampled(name):
    require_gpu()
    from test_gpu_ffn import _gpu_ffn
    w = _mx(name)
    x, _ = synth.make_tokens(w)
    ids, wt = _routing(w, x)
    y = _gpu_ffn(w, x, ids, wt, "prefill")
    rows = _sample_rows(ids, w.E, 56, 2)
    assert len(rows) >= 64
    assert_close_rms(y[rows], _oracle_rows(w, x, ids, wt, rows), what=f"mxfp4 {name} {len(rows)} sampled tokens")
    assert np.all(np.isfinite(y))


@pytest.mark.parametrize("T", [1, 16])
def test_forward_decode_routes_and_matches_oracle(T):
    require_gpu()
    import bit_moe_amd as bm
    w0 = _mx("decode_b1")
    w = w0.with_(T=T, name=f"mx_fwd{T}")
    L = synth_layer(w0)
    x, _ = synth.make_tokens(w, accept=lambda t, r: oracle.margin_ok(r, L.router(), w.k, 1e-4))
    y, gid, gw = bm.forward_decode(device_layer(w0), x_to_device(x))
    torch.cuda.synchronize()
    rid, rw = oracle.route(x, L.router(), w.k)
    np.testing.assert_array_equal(gid.cpu().numpy(), rid)
    np.testing.assert_allclose(gw.cpu().numpy(), rw, atol=W_TOL)
    assert_close_rms(y.cpu().numpy(), oracle.layer_ffn(L, x, rid, rw), what=f"mxfp4 forward_decode T={T}")


def test_scale_bytes_far_from_the_generator_and_per_expert():
    """Each expert tensor's scale bytes shifted by its own offset in
    [-30, +30]: weights from about 2^-40 to 2^26, experts' outputs up to
    2^180 apart (within fp32 for every intermediate).  One expert per token
    (k = 1), so that every expert's own output is compared, relative to its
    own rms; decode and prefill against the oracle on the same blocks."""
    require_gpu()
    import bit_moe_amd as bm
    w = _mx("tiny").with_(name="tiny_mx_env", T=37, x_dtype="bf16", seed=52)
    L = synth_layer(w)
    rng = np.random.default_rng(9)
    tens = {}
    for name, fn in (("gate", L.gate), ("up", L.up), ("down", L.down)):
        d = {}
        for e in range(w.E):
            b = fn(e).copy()
            b[:, 0] = (b[:, 0].astype(np.int64) + int(rng.integers(-30, 31))).astype(np.uint8)
            d[e] = b
        tens[name] = d
    stack = lambda d: np.stack([d[e] for e in range(w.E)])
    lay = bm.layer_from_canonical(w.H, w.I, w.E, 1, L.router(), stack(tens["gate"]), stack(tens["up"]),
                                  stack(tens["down"]), None, None, fmt=bm.FORMAT_MXFP4)
    x, _ = synth.make_tokens(w)
    ids = (np.arange(w.T, dtype=np.int32) % w.E).reshape(-1, 1)
    wt = np.ones((w.T, 1), np.float32)
    ref = oracle.moe_ffn(w.H, w.I, w.E, 1, None, tens["gate"], tens["up"], tens["down"], None, x, ids,
                         wt.astype(np.float64), fmt="mxfp4")
    rms = np.sqrt(np.mean(ref ** 2, axis=1))
    say(f"[mxfp4] envelope: per-token output rms from {rms.min():.2e} to {rms.max():.2e}")
    assert np.all(np.isfinite(ref)) and np.all(rms > 0)
    for mode, fn in (("decode", bm.ffn_decode), ("prefill", bm.ffn_prefill)):
        y = fn(lay, x_to_device(x), torch.from_numpy(ids).cuda(), torch.from_numpy(wt).cuda())
        torch.cuda.synchronize()
        y = y.cpu().numpy().astype(np.float64)
        assert np.all(np.isfinite(y))
        ratio = np.max(np.abs(y - ref), axis=1) / rms
        say(f"[parity] mxfp4 scale envelope/{mode}: worst token max|err|/rms = {ratio.max():.3e}")
        assert ratio.max() <= 2e-2, (mode, int(np.argmax(ratio)))
