"""GPU: the build that checks the caller's routing ids (BITMOE_CHECK_IDS=1,
libbitmoe_checked.so).

With valid ids its outputs are the release build's bit for bit (the clamp
leaves valid ids as they are) and the count at the start of the workspace
is 0.  With ids outside [0, E) the count is theirs and the call stays in
bounds: every id is read clamped into range, so the output is finite (and
wrong for the tokens concerned).  The bad ids are placed so that no row
repeats an expert after the clamp.  Cases: decode of one token (ids given
to the single-token path), of 5 tokens (one launch for all experts, wave
bucketing), of 37 tokens (prefill kernels beside the decode ones); prefill
of 37 tokens (single-block bucketing) and of 2100 tokens (multi-block
bucketing); moe_bucket alone."""
import numpy as np
import pytest

import synth
from _gpu import device_layer, require_gpu, say, torch, x_to_device

pytestmark = pytest.mark.gpu


def _ids_and_weights(T, E, k, seed):
    rng = np.random.default_rng(seed)
    ids = np.stack([rng.choice(E, size=k, replace=False) for _ in range(T)]).astype(np.int32)
    w = rng.random((T, k)).astype(np.float32)
    return ids, w / w.sum(axis=1, keepdims=True)


def _spoil(ids, E, n_bad, seed):
    """n_bad ids replaced by values outside [0, E) whose clamp (0 or E - 1)
    is not already in the row."""
    rng = np.random.default_rng(seed)
    bad = ids.copy()
    done = 0
    for t in rng.permutation(ids.shape[0]):
        if done == n_bad:
            break
        row = set(int(v) for v in bad[t])
        j = int(rng.integers(ids.shape[1]))
        rest = row - {int(bad[t, j])}
        if 0 not in rest:
            bad[t, j] = -1 - int(rng.integers(1000))
        elif E - 1 not in rest:
            bad[t, j] = E + int(rng.integers(1000))
        else:
            continue
        done += 1
    assert done == n_bad
    return bad


def _flag(ws):
    return int(ws[:4].view(torch.int32).item())


@pytest.mark.parametrize("mode,T", [("decode", 1), ("decode", 5), ("decode", 37), ("prefill", 37),
                                    ("prefill", 2100)])
def test_checked_build_counts_bad_ids_and_matches_release(mode, T):
    require_gpu()
    import bit_moe_amd as bm
    checked = bm.lib_checked()
    assert "checked" in checked.moe_version().decode() and "checked" not in bm.version()
    w = synth.WORKLOADS["tiny"].with_(name=f"tiny_chk_{T}", T=T, shared=True, x_dtype="bf16", seed=90)
    lay = device_layer(w)
    x, _ = synth.make_tokens(w)
    xd = x_to_device(x)
    ids, wt = _ids_and_weights(T, w.E, w.k, 7 + T)
    fn = bm.ffn_decode if mode == "decode" else bm.ffn_prefill
    nbytes = bm.workspace_bytes(lay, T, bm.DECODE if mode == "decode" else bm.PREFILL)
    wd = torch.from_numpy(wt).cuda()
    ws = torch.full((nbytes,), 0x5A, dtype=torch.uint8, device="cuda")
    y_rel = fn(lay, xd, torch.from_numpy(ids).cuda(), wd)
    y_chk = fn(lay, xd, torch.from_numpy(ids).cuda(), wd, ws=ws, library=checked)
    torch.cuda.synchronize()
    assert _flag(ws) == 0
    np.testing.assert_array_equal(y_chk.cpu().numpy().view(np.uint32), y_rel.cpu().numpy().view(np.uint32))
    n_bad = max(1, min(T // 2, 9))
    bad = _spoil(ids, w.E, n_bad, 11 + T)
    y_bad = fn(lay, xd, torch.from_numpy(bad).cuda(), wd, ws=ws, library=checked)
    torch.cuda.synchronize()
    assert _flag(ws) == n_bad
    assert np.all(np.isfinite(y_bad.cpu().numpy()))
    say(f"[checked ids] {mode} T={T}: valid ids bit-identical to the release build, {n_bad} bad ids counted")


def test_checked_bucket_counts_bad_ids():
    require_gpu()
    import bit_moe_amd as bm
    E, k, T = 64, 2, 3000                   # 6000 pairs: the multi-block bucketing
    ids, _ = _ids_and_weights(T, E, k, 3)
    bad = _spoil(ids, E, 17, 4)
    checked = bm.lib_checked()
    ws = torch.full((checked.moe_bucket_workspace_bytes(T, k, E),), 0x5A, dtype=torch.uint8, device="cuda")
    dev = torch.from_numpy(bad).cuda()
    counts = torch.empty(E, dtype=torch.int32, device="cuda")
    offsets = torch.empty(E + 1, dtype=torch.int32, device="cuda")
    perm = torch.empty(T * k, dtype=torch.int32, device="cuda")
    active = torch.empty(E, dtype=torch.int32, device="cuda")
    n_active = torch.empty(1, dtype=torch.int32, device="cuda")
    rc = checked.moe_bucket(dev.data_ptr(), T, k, E, counts.data_ptr(), offsets.data_ptr(), perm.data_ptr(),
                            active.data_ptr(), n_active.data_ptr(), ws.data_ptr(), ws.numel(), None)
    torch.cuda.synchronize()
    assert rc == 0
    assert _flag(ws) == 17
    # every pair lands in some expert's bucket (the bad ones in the clamped one)
    assert int(counts.sum().item()) == T * k
    assert sorted(perm.cpu().numpy().tolist()) == list(range(T * k))
