"""Pins of the oracle's quantizer round trip (CPU only, oracle/quant.c).

The pages name the formats and say the quantisation is asymmetric and
importance-weighted, but print no algorithm, example or error figure, so the
encoder is this build's reading: an unweighted squared-error search over
each format's own choices.  It is pinned by what that definition fixes:
 - blocks whose values the format represents exactly come back exactly
   (zero error is reachable, and the search finds it);
 - every IQ2X group choice is the brute-force optimum over all group scales,
   codebook rows and the 128 even-parity sign patterns of each run;
 - every Q2K sub-block choice is the brute-force optimum over its searched
   3 x 3 window of (scale, min) codes, and never worse than the window's
   centre;
 - all-zero superblocks encode to zero bytes.
The brute force here is numpy over the decoded values, written from the
format description; it shares nothing with quant.c.
"""
import numpy as np
import pytest

import oracle
import synth

GRID = synth.make_layer(synth.WORKLOADS["tiny"]).grid()


def _f16(v):
    return np.array(v, dtype=np.float16).view(np.uint16)


def _iq2x_representable(rng, n):
    """Random IQ2X blocks whose largest value is d * 27.125 (group scale 15,
    magnitude 7 on weight 0), so the encoder's d equals the block's."""
    blk = rng.integers(0, 256, size=(n, 66), dtype=np.uint8)
    rows7 = np.nonzero(GRID[:, 0] == 7)[0]
    for b in range(n):
        d = np.float16(np.exp2(rng.uniform(-16, -6)))
        blk[b, 0:2] = np.array([d]).view(np.uint8)
        a = int.from_bytes(bytes(blk[b, 6:10]), "little") | (15 << 28)
        blk[b, 6:10] = np.frombuffer(a.to_bytes(4, "little"), dtype=np.uint8)
        blk[b, 2] = rows7[b % len(rows7)]
    return blk


def test_iq2x_exact_round_trip_of_representable_blocks():
    rng = np.random.default_rng(11)
    blk = _iq2x_representable(rng, 24)
    w = oracle.dequant_iq2x(blk, GRID)
    assert np.all(w.astype(np.float32).astype(np.float64) == w)      # exact in fp32
    re = oracle.quantize_iq2x(w.astype(np.float32), GRID)
    np.testing.assert_array_equal(oracle.dequant_iq2x(re, GRID), w)
    np.testing.assert_array_equal(re[:, 0:2], blk[:, 0:2])           # same d


def _q2k_representable(rng, n):
    """Random Q2K blocks with d and dmin of one binade (so every value is
    exact in fp32), sub-block scale codes 1..15 with sub-block 0 at (15, 15),
    and quants 0 and 3 in every sub-block (so each sub-block's min and range
    give back its codes)."""
    blk = np.zeros((n, 84), dtype=np.uint8)
    for b in range(n):
        e = rng.integers(-14, -6)
        d, dm = (np.float16(np.exp2(e) * rng.uniform(1, 2)) for _ in range(2))
        blk[b, 80:82] = np.array([d]).view(np.uint8)
        blk[b, 82:84] = np.array([dm]).view(np.uint8)
        sc = rng.integers(1, 16, 16)
        mn = rng.integers(0, 16, 16)
        sc[0] = mn[0] = 15
        blk[b, 0:16] = sc | (mn << 4)
        q = rng.integers(0, 4, 256)
        q[0::16], q[1::16] = 0, 3
        for i in range(256):
            h, r = divmod(i, 128)
            j, l = divmod(r, 32)
            blk[b, 16 + 32 * h + l] |= q[i] << (2 * j)
    return blk


def test_q2k_exact_round_trip_of_representable_blocks():
    rng = np.random.default_rng(12)
    blk = _q2k_representable(rng, 24)
    w = oracle.dequant_q2k(blk)
    assert np.all(w.astype(np.float32).astype(np.float64) == w)
    re = oracle.quantize_q2k(w.astype(np.float32))
    np.testing.assert_array_equal(oracle.dequant_q2k(re), w)
    np.testing.assert_array_equal(re[:, 80:84], blk[:, 80:84])       # same d, dmin


def _even_sign_patterns():
    p = np.arange(256)
    bits = (p[:, None] >> np.arange(8)) & 1
    return np.where(bits[bits.sum(axis=1) % 2 == 0] == 1, -1.0, 1.0)   # [128, 8]


def test_iq2x_groups_are_brute_force_optimal():
    """For each group: the least squared error over all 16 scales x 256 rows
    x 128 even-parity sign patterns per run equals the encoder's error."""
    rng = np.random.default_rng(13)
    w = (rng.standard_normal(256 * 3) * np.exp2(rng.integers(-8, 0, 256 * 3))).astype(np.float32)
    blk = oracle.quantize_iq2x(w, GRID)
    got = oracle.dequant_iq2x(blk, GRID)
    signs = _even_sign_patterns()
    g = GRID.astype(np.float64)
    for b in range(blk.shape[0]):
        d = float(blk[b, 0:2].view(np.float16)[0])
        wb = w[256 * b:256 * (b + 1)].astype(np.float64)
        assert d == float(np.float16(np.abs(wb).max() / 27.125))
        for grp in range(8):
            best = np.inf
            for s in range(16):
                db = d * (0.5 + s) / 4
                tot = 0.0
                for j in range(4):
                    x = wb[32 * grp + 8 * j: 32 * grp + 8 * j + 8]
                    v = db * g[:, None, :] * signs[None, :, :]             # [256, 128, 8]
                    tot += ((x - v) ** 2).sum(axis=2).min()
                best = min(best, tot)
            sl = slice(256 * b + 32 * grp, 256 * b + 32 * grp + 32)
            mine = ((got[sl] - w[sl].astype(np.float64)) ** 2).sum()
            assert mine == pytest.approx(best, rel=1e-12, abs=1e-300), (b, grp)


def test_q2k_sub_blocks_are_window_optimal_and_never_worse_than_start():
    rng = np.random.default_rng(14)
    w = (rng.standard_normal(256 * 6) * 0.03 + rng.uniform(-0.01, 0.01, 256 * 6)).astype(np.float32)
    blk = oracle.quantize_q2k(w)
    got = oracle.dequant_q2k(blk)
    for b in range(blk.shape[0]):
        d = float(blk[b, 80:82].view(np.float16)[0])
        dm = float(blk[b, 82:84].view(np.float16)[0])
        wb = w[256 * b:256 * (b + 1)].astype(np.float64).reshape(16, 16)
        m = np.where(wb.min(axis=1) < 0, -wb.min(axis=1), 0.0)
        a = np.where(wb.max(axis=1) + m > 0, (wb.max(axis=1) + m) / 3, 0.0)
        assert d == float(np.float16(a.max() / 15)) and dm == float(np.float16(m.max() / 15))

        def err(sb, cs, cm):
            A, M = d * cs, dm * cm
            q = np.clip(np.rint((wb[sb] + M) / A), 0, 3) if A > 0 else np.zeros(16)
            return ((wb[sb] - (A * q - M)) ** 2).sum()
        for sb in range(16):
            cs0 = int(np.clip(np.rint(a[sb] / d), 0, 15)) if d > 0 else 0
            cm0 = int(np.clip(np.rint(m[sb] / dm), 0, 15)) if dm > 0 else 0
            window = [err(sb, cs, cm) for cs in range(cs0 - 1, cs0 + 2) for cm in range(cm0 - 1, cm0 + 2)
                      if 0 <= cs <= 15 and 0 <= cm <= 15]
            mine = ((got[256 * b + 16 * sb: 256 * b + 16 * sb + 16] - wb[sb]) ** 2).sum()
            assert mine == pytest.approx(min(window), rel=1e-12, abs=1e-300)
            assert mine <= err(sb, cs0, cm0) * (1 + 1e-12)


def test_all_zero_superblocks_encode_to_zero_bytes():
    z = np.zeros(512, dtype=np.float32)
    assert not oracle.quantize_iq2x(z, GRID).any()
    assert not oracle.quantize_q2k(z).any()


def test_error_on_gaussian_weights_is_that_of_two_bits():
    """Relative rms error on N(0, 1) weights: about 0.37 (IQ2X, 2.06 bits
    per weight with this random codebook) and 0.28 (Q2K, 2.625 bits)."""
    rng = np.random.default_rng(15)
    w = rng.standard_normal(256 * 64).astype(np.float32)
    ei = np.sqrt(np.mean((oracle.dequant_iq2x(oracle.quantize_iq2x(w, GRID), GRID) - w) ** 2))
    eq = np.sqrt(np.mean((oracle.dequant_q2k(oracle.quantize_q2k(w)) - w) ** 2))
    assert 0.25 < ei < 0.45 and 0.2 < eq < 0.35, (ei, eq)


# ---- MXFP4 (OCP Microscaling conversion with a two-way scale search) --------

E2M1 = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0, -0.0, -0.5, -1.0, -1.5, -2.0, -3.0, -4.0, -6.0])


def test_mxfp4_exact_round_trip_of_representable_blocks():
    """Random codes at a random scale with one element at +-6: the shared
    exponent floor(log2 6 s) - 2 is the block's own, so every value comes back."""
    rng = np.random.default_rng(21)
    n = 64
    blk = rng.integers(0, 256, size=(n, 17), dtype=np.uint8)
    blk[:, 0] = rng.integers(20, 235, n)
    blk[:, 1] = (blk[:, 1] & 0xF0) | rng.choice([7, 15], n)          # element 0: +-6
    w = oracle.dequant_mxfp4(blk)
    assert np.all(w.astype(np.float32).astype(np.float64) == w)
    re = oracle.quantize_mxfp4(w.astype(np.float32))
    np.testing.assert_array_equal(oracle.dequant_mxfp4(re), w)       # (-0 and +0 compare equal)
    np.testing.assert_array_equal(re[:, 0], blk[:, 0])


def test_mxfp4_blocks_are_optimal_over_the_two_scales():
    """For each block: the scale byte is e0 + 127 or e0 + 128 (e0 = floor(log2
    max|w|) - 2), and the squared error equals the brute-force minimum over
    those two scales and all 16 codes of every element."""
    rng = np.random.default_rng(22)
    w = (rng.standard_normal(32 * 200) * np.exp2(rng.integers(-20, 20, 32 * 200))).astype(np.float32)
    blk = oracle.quantize_mxfp4(w)
    got = oracle.dequant_mxfp4(blk).reshape(-1, 32)
    wb = w.astype(np.float64).reshape(-1, 32)
    for b in range(blk.shape[0]):
        e0 = int(np.floor(np.log2(np.abs(wb[b]).max()))) - 2
        assert int(blk[b, 0]) - 127 in (e0, e0 + 1)
        best = min(((wb[b][:, None] - E2M1[None, :] * 2.0 ** e) ** 2).min(axis=1).sum() for e in (e0, e0 + 1))
        mine = ((got[b] - wb[b]) ** 2).sum()
        assert mine == pytest.approx(best, rel=1e-12, abs=1e-300), b


def test_mxfp4_element_ties_round_to_even_mantissa():
    """Midpoints between E2M1 values at scale 1 (kept by the exactly
    representable 6, 0.5 and 1.5 elsewhere in the block): 0.25 -> 0,
    0.75 -> 1, 1.25 -> 1, 1.75 -> 2, 2.5 -> 2, 3.5 -> 4, 5 -> 4, and their
    negatives."""
    ties = [0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0]
    want = [0.0, 1.0, 1.0, 2.0, 2.0, 4.0, 4.0]
    w = np.array([6.0] + ties + [-t for t in ties] + [0.5, 1.5] * 8 + [0.5], dtype=np.float32)[:32]
    blk = oracle.quantize_mxfp4(w)
    assert blk[0, 0] == 127
    got = oracle.dequant_mxfp4(blk)
    np.testing.assert_array_equal(got[1:8], want)
    np.testing.assert_array_equal(got[8:15], [-v for v in want])


def test_mxfp4_zero_blocks_and_gaussian_error():
    assert not oracle.quantize_mxfp4(np.zeros(64, np.float32)).any()
    rng = np.random.default_rng(23)
    w = rng.standard_normal(32 * 512).astype(np.float32)
    e = np.sqrt(np.mean((oracle.dequant_mxfp4(oracle.quantize_mxfp4(w)) - w) ** 2))
    assert 0.08 < e < 0.15, e
