"""GPU: repeated decode calls that share one workspace.

The decode launches hand results between workgroups of one launch (router
logits to the routing workgroup, per-panel down outputs to the combining
workgroup) through device-scope stores and per-call flags.  Stale data from
an earlier call would show up as a wrong output, so every call of a long
run with changing batches is checked against the oracle."""
import numpy as np
import pytest

import oracle
import synth
from _gpu import assert_close_rms, require_gpu, say, synth_layer, torch, x_to_device

pytestmark = pytest.mark.gpu

W = synth.Workload("handover", 1, 2048, 512, 64, 8, "bf16", "computed", None, True, 31, "decode")


def test_many_calls_one_workspace_forward_and_given_ids():
    require_gpu()
    import bit_moe_amd as bm
    L = synth_layer(W)
    lay = bm.layer_from_canonical(W.H, W.I, W.E, W.k, L.router(), L.gate_all(), L.up_all(),
                                  L.down_all(), L.grid(), L.shared())
    pool, _ = synth.make_tokens(W.with_(T=160),
                                accept=lambda t, r: oracle.margin_ok(r, L.router(), W.k, 1e-4))
    sizes = [1, 3, 16, 8, 1, 16, 2, 5, 1, 16, 11, 1, 4, 16, 7, 1]
    ws = torch.empty(bm.workspace_bytes(lay, 16, bm.DECODE), dtype=torch.uint8, device="cuda")
    t0 = 0
    for i, T in enumerate(sizes):
        x = pool[t0:t0 + T]
        t0 = (t0 + T) % (pool.shape[0] - 16)
        rid, rw = oracle.route(x, L.router(), W.k)
        ref = oracle.layer_ffn(L, x, rid, rw)
        if i % 2 == 0:
            y, gid, gw = bm.forward_decode(lay, x_to_device(x), ws=ws)
            torch.cuda.synchronize()
            np.testing.assert_array_equal(gid.cpu().numpy(), rid)
        else:
            ids = torch.from_numpy(rid.astype(np.int32)).cuda()
            wt = torch.from_numpy(rw.astype(np.float32)).cuda()
            y = bm.ffn_decode(lay, x_to_device(x), ids, wt, ws=ws)
            torch.cuda.synchronize()
        say(f"[handover] call {i} T={T} {'forward' if i % 2 == 0 else 'given ids'}")
        assert_close_rms(y.cpu().numpy(), ref, what=f"call {i} T={T}")
