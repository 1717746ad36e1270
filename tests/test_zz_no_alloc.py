"""GPU: moe_forward_decode_noalloc (the decode step with the library's
static scratch, for callers that cannot allocate) against
moe_forward_decode with a caller workspace, through the C ABI.  Two calls
in a row on each layer, the second with fewer tokens, so the second runs on
an array that still holds the first call's contents."""
import numpy as np
import pytest

import oracle
import synth
from _gpu import W_TOL, assert_close_rms, device_layer, require_gpu, say, synth_layer, torch, x_to_device

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("name,sizes", [("decode_b1", (16, 1)), ("tiny_shared_f32", (7, 3))])
def test_noalloc_matches_workspace_entry_point(name, sizes):
    require_gpu()
    import bit_moe_amd as bm
    if name == "decode_b1":
        w0 = synth.WORKLOADS["decode_b1"]
    else:
        w0 = synth.WORKLOADS["tiny"].with_(name="tiny_na", shared=True, x_dtype="f32", seed=61)
    L = synth_layer(w0)
    lay = device_layer(w0)
    for T in sizes:
        w = w0.with_(T=T, name=f"{w0.name}_na{T}")
        x, _ = synth.make_tokens(w, accept=lambda t, r: oracle.margin_ok(r, L.router(), w.k, 1e-4))
        xd = x_to_device(x)
        say(f"[noalloc] {name} T={T}")
        y_ref, id_ref, w_ref = bm.forward_decode(lay, xd)
        y_na, id_na, w_na = bm.forward_decode_noalloc(lay, xd)
        torch.cuda.synchronize()
        np.testing.assert_array_equal(id_na.cpu().numpy(), id_ref.cpu().numpy())
        np.testing.assert_allclose(w_na.cpu().numpy(), w_ref.cpu().numpy(), rtol=0, atol=W_TOL)
        same = bool(torch.equal(y_na, y_ref))
        say(f"[noalloc] {name} T={T} bit-identical to the workspace call: {same}")
        assert_close_rms(y_na.cpu().numpy(), y_ref.cpu().numpy().astype(np.float64),
                         what=f"noalloc vs workspace {name} T={T}")
