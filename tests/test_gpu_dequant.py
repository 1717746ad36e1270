"""GPU parity: standalone dequantisation (bit-exact against the oracle).

Each value is exact in fp32 (IQ2X) or one fp32 rounding of an exact value
(Q2K), so the fp32 output must equal float32(oracle) bit for bit, and the
bf16 output must equal the round-to-nearest-even of that fp32 value."""
import json
import os

import numpy as np
import pytest

import oracle
import synth
from _gpu import require_gpu, say, torch

pytestmark = pytest.mark.gpu
GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _gpu_iq2x(blocks, grid, out_dtype):
    import bit_moe_amd as bm
    b = torch.from_numpy(np.ascontiguousarray(blocks).reshape(-1)).cuda()
    g = torch.from_numpy(np.ascontiguousarray(grid).reshape(-1)).cuda()
    out = bm.dequant_iq2x(b, g, out_dtype)
    torch.cuda.synchronize()
    return out


def _gpu_q2k(blocks, out_dtype):
    import bit_moe_amd as bm
    b = torch.from_numpy(np.ascontiguousarray(blocks).reshape(-1)).cuda()
    out = bm.dequant_q2k(b, out_dtype)
    torch.cuda.synchronize()
    return out


def _check_f32(out, ref64):
    got = out.cpu().numpy()
    exp = ref64.astype(np.float32)
    np.testing.assert_array_equal(got.view(np.uint32), exp.view(np.uint32))


def _check_bf16(out, ref64):
    got = out.view(torch.int16).cpu().numpy().view(np.uint16)
    exp = synth.bf16_bits_from_f32(ref64.astype(np.float32))
    np.testing.assert_array_equal(got, exp)


def _random_blocks(n, size, dofs, seed):
    rng = np.random.default_rng(seed)
    b = rng.integers(0, 256, size=(n, size), dtype=np.uint8)
    # any finite fp16 for d (and dmin): normals, subnormals, negatives, zero
    for o in dofs:
        h = rng.integers(0, 1 << 16, size=n, dtype=np.uint16)
        h[(h & 0x7C00) == 0x7C00] &= 0x83FF          # keep finite
        b[:, o] = h & 0xFF
        b[:, o + 1] = h >> 8
    return b


@pytest.mark.parametrize("out_dtype", [0, 1])
def test_iq2x_random_blocks(out_dtype):
    require_gpu()
    b = _random_blocks(20000, 66, [0], 1)
    grid = (2 * np.random.default_rng(2).integers(0, 4, size=(256, 8)) + 1).astype(np.uint8)
    ref = oracle.dequant_iq2x(b, grid)
    out = _gpu_iq2x(b, grid, out_dtype)
    (_check_bf16 if out_dtype else _check_f32)(out, ref)


@pytest.mark.parametrize("out_dtype", [0, 1])
def test_q2k_random_blocks(out_dtype):
    require_gpu()
    b = _random_blocks(20000, 84, [80, 82], 3)
    ref = oracle.dequant_q2k(b)
    out = _gpu_q2k(b, out_dtype)
    (_check_bf16 if out_dtype else _check_f32)(out, ref)


def test_hand_built_golden_blocks():
    require_gpu()
    g = json.load(open(os.path.join(GOLDEN, "iq2x_hand.json")))
    grid = np.tile(np.array(g["grid_default_row"], dtype=np.uint8), (256, 1))
    for r, row in g["grid_rows"].items():
        grid[int(r)] = row
    blocks = np.stack([np.frombuffer(bytes.fromhex(c["hex"].replace(" ", "")), dtype=np.uint8)
                       for c in g["cases"]])
    _check_f32(_gpu_iq2x(blocks, grid, 0), oracle.dequant_iq2x(blocks, grid))
    q = json.load(open(os.path.join(GOLDEN, "q2k_hand.json")))
    qb = np.stack([np.frombuffer(bytes.fromhex(c["hex"].replace(" ", "")), dtype=np.uint8)
                   for c in q["cases"]])
    _check_f32(_gpu_q2k(qb, 0), oracle.dequant_q2k(qb))


@pytest.mark.parametrize("name", ["tiny", "decode_b1"])
def test_layer_tensors_bit_exact(name):
    """One whole expert of each projection at the workload's real shape."""
    require_gpu()
    w = synth.WORKLOADS[name]
    L = synth.make_layer(w)
    for e in (0, w.E - 1):
        say(f"[dequant] {name} expert {e}")
        for blk in (L.gate(e), L.up(e)):
            ref = oracle.dequant_iq2x(blk, L.grid())
            _check_f32(_gpu_iq2x(blk, L.grid(), 0), ref)
            _check_bf16(_gpu_iq2x(blk, L.grid(), 1), ref)
        ref = oracle.dequant_q2k(L.down(e))
        _check_f32(_gpu_q2k(L.down(e), 0), ref)
        _check_bf16(_gpu_q2k(L.down(e), 1), ref)


def test_empty_and_single_block():
    require_gpu()
    import bit_moe_amd as bm
    z = torch.zeros(0, dtype=torch.uint8, device="cuda")
    g = torch.ones(2048, dtype=torch.uint8, device="cuda")
    assert bm.dequant_iq2x(z, g).numel() == 0
    assert bm.dequant_q2k(z).numel() == 0
    b = _random_blocks(1, 66, [0], 9)
    grid = np.ones((256, 8), dtype=np.uint8) * 3
    _check_f32(_gpu_iq2x(b, grid, 0), oracle.dequant_iq2x(b, grid))
