"""Pins of the oracle's dequantisation (CPU only).

The pages print no worked example of either block format, so the oracle's
decoders are pinned by: hand-decoded golden blocks (tests/golden/), the fp16
decoding against numpy's IEEE half type for all 65536 patterns, invariants
that hold for any correct decoder on random blocks, and an independent numpy
decoder (below) that must agree bit for bit on every tiny-config tensor and
on 2^20 random superblocks of each format.
"""
import json
import os

import numpy as np
import pytest

import oracle
import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _expand(spec):
    out = []
    for item in spec:
        if item[0] == "repeat":
            _, n, inner = item
            out += _expand(inner) * n
        else:
            cnt, expr = item
            out += [float(eval(expr, {"__builtins__": {}}))] * cnt
    return out


def _golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def _hand_grid(g):
    grid = np.tile(np.array(g["grid_default_row"], dtype=np.uint8), (256, 1))
    for r, row in g["grid_rows"].items():
        grid[int(r)] = row
    return grid


@pytest.mark.parametrize("case", [c["name"] for c in _golden("iq2x_hand.json")["cases"]])
def test_iq2x_golden(case):
    g = _golden("iq2x_hand.json")
    c = next(c for c in g["cases"] if c["name"] == case)
    blk = np.frombuffer(bytes.fromhex(c["hex"].replace(" ", "")), dtype=np.uint8)
    assert blk.size == 66
    exp = np.array(_expand(c["expect"]))
    assert exp.size == 256
    got = oracle.dequant_iq2x(blk, _hand_grid(g))
    np.testing.assert_array_equal(got, exp)


@pytest.mark.parametrize("case", [c["name"] for c in _golden("q2k_hand.json")["cases"]])
def test_q2k_golden(case):
    c = next(c for c in _golden("q2k_hand.json")["cases"] if c["name"] == case)
    blk = np.frombuffer(bytes.fromhex(c["hex"].replace(" ", "")), dtype=np.uint8)
    assert blk.size == 84
    exp = np.array(_expand(c["expect"]))
    assert exp.size == 256
    np.testing.assert_array_equal(oracle.dequant_q2k(blk), exp)


def test_fp16_decode_all_patterns():
    """Every binary16 pattern decodes as numpy's IEEE half type does."""
    pats = np.arange(65536, dtype=np.uint16)
    ref = pats.view(np.float16).astype(np.float64)
    got = np.array([oracle.fp16_to_double(int(p)) for p in pats])
    fin = np.isfinite(ref)
    np.testing.assert_array_equal(got[fin], ref[fin])
    np.testing.assert_array_equal(np.isnan(got), np.isnan(ref))
    np.testing.assert_array_equal(np.isinf(got) & (got > 0), np.isinf(ref) & (ref > 0))


def _random_iq2x(n, seed):
    rng = np.random.default_rng(seed)
    b = rng.integers(0, 256, size=(n, 66), dtype=np.uint8)
    b[:, 0:2] = np.asarray(rng.uniform(0.01, 2.0, n), dtype=np.float16).view(np.uint8).reshape(-1, 2)
    grid = (2 * rng.integers(0, 4, size=(256, 8)) + 1).astype(np.uint8)
    return b, grid


def test_iq2x_invariants_random_blocks():
    """For any block: each run of 8 has an even number of negative values;
    |v| / grid magnitude is the same for the 32 values of a group; and the 8
    group ratios over d take the 16 admissible values (0.5+s)/4."""
    b, grid = _random_iq2x(4000, 11)
    v = oracle.dequant_iq2x(b, grid).reshape(-1, 8, 4, 8)          # block, group, sub, i
    idx = b[:, 2:].reshape(-1, 8, 8)[:, :, :4]                      # block, group, sub
    mag = grid[idx].astype(np.float64)                              # block, group, sub, i
    neg = (v < 0).sum(axis=-1)
    assert np.all(neg % 2 == 0)
    ratio = np.abs(v) / mag
    assert np.all(ratio == ratio[:, :, :1, :1])
    d = b[:, 0:2].copy().view(np.float16).astype(np.float64).reshape(-1, 1)
    r = ratio[:, :, 0, 0] / d
    admissible = (0.5 + np.arange(16)) / 4
    assert np.all(np.isin(r, admissible))
    # the 4-bit scale lives in the top nibble of the group's last byte
    s = b[:, 2:].reshape(-1, 8, 8)[:, :, 7] >> 4
    np.testing.assert_array_equal(r, (0.5 + s) / 4)


def test_iq2x_sign_flip_of_one_bit():
    """Flipping one stored sign bit negates exactly two values of that run:
    the flipped one and the parity-carrying eighth."""
    b, grid = _random_iq2x(50, 5)
    base = oracle.dequant_iq2x(b, grid)
    rng = np.random.default_rng(0)
    for blk in range(50):
        g, j, i = rng.integers(0, 8), rng.integers(0, 4), rng.integers(0, 7)
        bit = 7 * j + i
        b2 = b.copy()
        b2[blk, 2 + 8 * g + 4 + bit // 8] ^= np.uint8(1 << (bit % 8))
        v = oracle.dequant_iq2x(b2, grid)
        diff = np.nonzero(v != base)[0]
        pos = blk * 256 + 32 * g + 8 * j
        assert sorted(diff.tolist()) == [pos + i, pos + 7]
        np.testing.assert_array_equal(v[diff], -base[diff])


def test_q2k_invariants_random_blocks():
    """Within a sub-block of 16 the values lie on q*d*scale - dmin*min with
    q in {0,1,2,3}; qs=0 gives -dmin*min; results are exact fp32 roundings."""
    rng = np.random.default_rng(3)
    n = 3000
    b = rng.integers(0, 256, size=(n, 84), dtype=np.uint8)
    b[:, 80:82] = np.asarray(rng.uniform(0.01, 1, n), dtype=np.float16).view(np.uint8).reshape(-1, 2)
    b[:, 82:84] = np.asarray(rng.uniform(0.01, 1, n), dtype=np.float16).view(np.uint8).reshape(-1, 2)
    v = oracle.dequant_q2k(b).reshape(n, 16, 16)
    d = b[:, 80:82].copy().view(np.float16).astype(np.float64).reshape(n, 1, 1)
    dm = b[:, 82:84].copy().view(np.float16).astype(np.float64).reshape(n, 1, 1)
    sc = (b[:, :16] & 0xF).astype(np.float64).reshape(n, 16, 1)
    mn = (b[:, :16] >> 4).astype(np.float64).reshape(n, 16, 1)
    q = (v + dm * mn)
    with np.errstate(invalid="ignore", divide="ignore"):
        qq = q / (d * sc)
    ok = (sc[..., 0] > 0)
    assert np.all(np.isin(qq[ok], [0.0, 1.0, 2.0, 3.0]))
    assert np.all(q[~ok] == 0)
    # zero quant bytes -> -dmin*min everywhere
    b0 = b.copy()
    b0[:, 16:80] = 0
    v0 = oracle.dequant_q2k(b0).reshape(n, 16, 16)
    np.testing.assert_array_equal(v0, np.broadcast_to(-dm * mn, v0.shape))


def test_q2k_quant_position_map():
    """Setting one 2-bit quant to 1 (d=1, scale 1, min 0) lights exactly one
    weight, the one at 128*h + 32*j + l for byte 32*h + l, bits 2j..2j+1."""
    blk = np.zeros(84, dtype=np.uint8)
    blk[:16] = 1
    blk[80:82] = np.array([1.0], dtype=np.float16).view(np.uint8)
    for h in range(2):
        for j in range(4):
            for l in (0, 7, 31):
                b = blk.copy()
                b[16 + 32 * h + l] = 1 << (2 * j)
                v = oracle.dequant_q2k(b)
                assert np.nonzero(v)[0].tolist() == [128 * h + 32 * j + l]
                assert v[128 * h + 32 * j + l] == 1.0


def test_values_are_exact_in_fp32():
    """Both formats' values are exactly representable in fp32 (IQ2X) or are a
    single subtraction of two fp32-exact products (Q2K), so the fp32 result a
    GPU decoder must produce is unique."""
    w = synth.WORKLOADS["tiny"]
    L = synth.make_layer(w)
    v = oracle.dequant_iq2x(L.gate(0), L.grid())
    assert np.all(v.astype(np.float32).astype(np.float64) == v)
    blk = L.down(0)
    d = blk[:, 80:82].copy().view(np.float16).astype(np.float32)
    dm = blk[:, 82:84].copy().view(np.float16).astype(np.float32)
    p1 = (d * np.float32(15) * np.float32(3)).astype(np.float64)
    p2 = (dm * np.float32(15)).astype(np.float64)
    assert np.all(p1 == d.astype(np.float64) * 45) and np.all(p2 == dm.astype(np.float64) * 15)


def test_generator_scale_fields_finite_positive():
    w = synth.WORKLOADS["tiny"]
    L = synth.make_layer(w)
    for blk, offs in ((L.gate(1), (0,)), (L.up(2), (0,)), (L.down(3), (80, 82))):
        for o in offs:
            d = blk[:, o:o + 2].copy().view(np.float16).astype(np.float64)
            assert np.all(np.isfinite(d)) and np.all(d > 0)


def test_slab_equals_slice_of_full_tensor():
    w = synth.WORKLOADS["tiny"]
    L = synth.make_layer(w)
    full = L.down_all()
    per = w.H * (w.I // 256)
    np.testing.assert_array_equal(full[3 * per:4 * per], L.down(3))


# ---- an independent decoder, written in numpy from the byte description ----
# (the format text of include/bitmoe.h: GGML's IQ2_XXS and Q2_K block orders,
# as "antirez/ds4 - Moteur local d'inference DeepSeek V4 Flash pour Metal",
# section "Remerciements a llama.cpp et GGML" has ds4 keep them, with the
# synthetic codebook).  It shares no code with the oracle: whole-array bit
# slicing instead of per-value loops, fp16 fields through numpy's half type.

_POP7 = np.array([bin(v).count("1") & 1 for v in range(128)], dtype=np.uint8)


def _np_iq2x(blocks, grid):
    b = np.ascontiguousarray(blocks, dtype=np.uint8).reshape(-1, 66)
    n = b.shape[0]
    d = b[:, 0:2].copy().view(np.float16).astype(np.float64).reshape(n)
    groups = b[:, 2:66].reshape(n, 8, 8)                       # [block, group, byte]
    idx = groups[:, :, 0:4]                                    # [block, group, run]
    a = groups[:, :, 4:8].copy().view("<u4").reshape(n, 8).astype(np.uint64)
    scale = (a >> 28).astype(np.float64)                       # [block, group]
    s7 = np.stack([(a >> (7 * j)) & 0x7F for j in range(4)], axis=2).astype(np.uint8)
    sign_byte = s7 | (_POP7[s7] << 7)                          # even parity in bit 7
    neg = np.unpackbits(sign_byte[..., None], axis=-1, bitorder="little")   # [block, group, run, i]
    mag = grid.astype(np.float64)[idx]                         # [block, group, run, i]
    db = d[:, None] * (0.5 + scale) * 0.25                     # [block, group]
    with np.errstate(invalid="ignore"):
        v = db[:, :, None, None] * mag * np.where(neg == 1, -1.0, 1.0)
    return v.reshape(n * 256)                                  # position 32 g + 8 run + i


def _np_q2k(blocks):
    b = np.ascontiguousarray(blocks, dtype=np.uint8).reshape(-1, 84)
    n = b.shape[0]
    sc = (b[:, 0:16] & 15).astype(np.float64)                  # [block, sub-block]
    mn = (b[:, 0:16] >> 4).astype(np.float64)
    qs = b[:, 16:80].reshape(n, 2, 1, 32)                      # [block, half, -, l]
    shifts = (2 * np.arange(4, dtype=np.uint8)).reshape(1, 1, 4, 1)
    q = ((qs >> shifts) & 3).astype(np.float64).reshape(n, 16, 16)   # value 128 h + 32 j + l
    d = b[:, 80:82].copy().view(np.float16).astype(np.float64).reshape(n, 1, 1)
    dmin = b[:, 82:84].copy().view(np.float16).astype(np.float64).reshape(n, 1, 1)
    with np.errstate(invalid="ignore"):                        # Inf * 0 patterns give NaN
        v = d * sc[:, :, None] * q - dmin * mn[:, :, None]
    return v.reshape(n * 256)


def _same(a, b):
    """Equal as IEEE values (NaN matches NaN whatever its payload), and
    bit-identical wherever finite."""
    np.testing.assert_array_equal(a, b)
    f = np.isfinite(a)
    np.testing.assert_array_equal(a[f].view(np.uint64), b[f].view(np.uint64))


def test_numpy_decoder_agrees_on_every_tiny_tensor():
    """Both decoders on every block of the tiny config's gate, up and down
    tensors (all 8 experts)."""
    L = synth.make_layer(synth.WORKLOADS["tiny"])
    grid = L.grid()
    for name, arr in (("gate", L.gate_all()), ("up", L.up_all())):
        _same(_np_iq2x(arr, grid), oracle.dequant_iq2x(arr, grid))
    down = L.down_all()
    _same(_np_q2k(down), oracle.dequant_q2k(down))


@pytest.mark.parametrize("fmt", ["iq2x", "q2k"])
def test_numpy_decoder_agrees_on_a_million_random_superblocks(fmt):
    """2^20 superblocks of uniformly random bytes per format: every fp16
    scale pattern occurs (zero, subnormal, negative, Inf, NaN), with random
    codebooks."""
    rng = np.random.default_rng(1234 if fmt == "iq2x" else 4321)
    nbytes = 66 if fmt == "iq2x" else 84
    total, chunk = 1 << 20, 1 << 16
    for c in range(total // chunk):
        blocks = rng.integers(0, 256, size=(chunk, nbytes), dtype=np.uint8)
        if fmt == "iq2x":
            grid = rng.integers(0, 256, size=(256, 8), dtype=np.uint8)
            _same(_np_iq2x(blocks, grid), oracle.dequant_iq2x(blocks, grid))
        else:
            _same(_np_q2k(blocks), oracle.dequant_q2k(blocks))


def test_numpy_decoder_matches_hand_goldens():
    """The numpy decoder also reproduces the hand-decoded golden blocks, so
    the three (hand values, oracle, numpy) agree."""
    g = _golden("iq2x_hand.json")
    for c in g["cases"]:
        blk = np.frombuffer(bytes.fromhex(c["hex"].replace(" ", "")), dtype=np.uint8)
        np.testing.assert_array_equal(_np_iq2x(blk, _hand_grid(g)), np.array(_expand(c["expect"])))
    for c in _golden("q2k_hand.json")["cases"]:
        blk = np.frombuffer(bytes.fromhex(c["hex"].replace(" ", "")), dtype=np.uint8)
        np.testing.assert_array_equal(_np_q2k(blk), np.array(_expand(c["expect"])))
