"""GPU pack entry points against the tiled layout written out in numpy from
the header's description (an independent statement of the same layout)."""
import numpy as np
import pytest

import synth
from _gpu import require_gpu, torch

pytestmark = pytest.mark.gpu


def _tiled_iq2x_numpy(canon, N, K):
    nb = K // 256
    b = canon.reshape(N, nb, 66)
    d = b[:, :, 0:2]
    grp = b[:, :, 2:].reshape(N, nb, 8, 8)
    idx = grp[:, :, :, :4].astype(np.uint32)
    a = grp[:, :, :, 4:8].copy().view("<u4")[..., 0]
    runs = np.zeros((N, nb, 8, 4), dtype=np.uint32)
    for j in range(4):
        # index byte, then 7 sign bits with scale bit j on top
        runs[..., j] = idx[..., j] | (((a >> (7 * j)) & 0x7F) << 8) | (((a >> (28 + j)) & 1) << 15)
    words = np.zeros((N, nb, 8, 2), dtype=np.uint32)
    words[..., 0] = runs[..., 0] | (runs[..., 1] << 16)
    words[..., 1] = runs[..., 2] | (runs[..., 3] << 16)
    qs = words.astype("<u4").view(np.uint8).reshape(N, nb, 4, 16)       # 4 pieces of 16 bytes
    qs = qs.reshape(N // 64, 64, nb, 4, 16).transpose(0, 2, 3, 1, 4)     # [P][kb][c][r][16]
    dd = d.reshape(N // 64, 64, nb, 2).transpose(0, 2, 1, 3)             # [P][kb][r][2]
    return np.concatenate([qs.reshape(-1), dd.reshape(-1)])


def _tiled_q2k_numpy(canon, N, K):
    nb = K // 256
    b = canon.reshape(N // 64, 64, nb, 84).transpose(0, 2, 1, 3)         # [P][kb][r][84]
    qs = b[..., 16:80].astype(np.uint32)                                  # [P][kb][r][64]
    # quant of weight i: (qs[32*(i//128) + i%32] >> 2*((i%128)//32)) & 3
    i = np.arange(256)
    q = (qs[..., 32 * (i // 128) + i % 32] >> (2 * ((i % 128) // 32))) & 3  # [P][kb][r][256]
    q = q.reshape(q.shape[:-1] + (16, 16))                                # sub-block, weight t
    t = np.arange(16)
    # weight t of a sub-block at bits 8 ((t & 7) >> 1) + 4 (t & 1) + 2 (t >> 3)
    words = (q << (8 * ((t & 7) >> 1) + 4 * (t & 1) + 2 * (t >> 3))).sum(axis=-1).astype(np.uint32)
    pieces = words.reshape(N // 64, nb, 64, 4, 4).transpose(0, 1, 3, 2, 4)    # [P][kb][c][r][4]
    qs_t = np.ascontiguousarray(pieces.astype("<u4")).view(np.uint8)
    return np.concatenate([qs_t.reshape(-1), b[..., 0:16].reshape(-1), b[..., 80:84].reshape(-1)])


def test_pack_iq2x_and_q2k_match_documented_layout():
    require_gpu()
    import bit_moe_amd as bm
    w = synth.WORKLOADS["tiny"]
    L = synth.make_layer(w)
    for e in (0, 5):
        g = L.gate(e)
        got = bm.pack_iq2x(torch.from_numpy(g.reshape(-1)).cuda(), 1, w.I, w.H).cpu().numpy()
        np.testing.assert_array_equal(got, _tiled_iq2x_numpy(g, w.I, w.H))
        dn = L.down(e)
        got = bm.pack_q2k(torch.from_numpy(dn.reshape(-1)).cuda(), 1, w.H, w.I).cpu().numpy()
        np.testing.assert_array_equal(got, _tiled_q2k_numpy(dn, w.H, w.I))


def test_pack_bf16_layout():
    require_gpu()
    import bit_moe_amd as bm
    rng = np.random.default_rng(0)
    N, K = 128, 512
    m = rng.integers(0, 1 << 16, size=(N, K), dtype=np.uint16)
    got = bm.pack_bf16(torch.from_numpy(m.view(np.int16)).cuda().view(torch.bfloat16))
    got = got.view(torch.int16).cpu().numpy().view(np.uint16)
    ref = m.reshape(N // 64, 64, K // 8, 8).transpose(0, 2, 1, 3).reshape(N, K)
    np.testing.assert_array_equal(got, ref)
