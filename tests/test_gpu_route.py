"""GPU parity: routing (ids bit-exact, weights within 1e-6) and bucketing
(bit-exact counts, offsets, stable permutation and active list)."""
import numpy as np
import pytest

import oracle
import synth
from _gpu import near_tie_tokens, require_gpu, say, synth_layer, torch, x_to_device

pytestmark = pytest.mark.gpu


def _route_gpu(w, x, router_bits=None):
    import bit_moe_amd as bm
    L = synth_layer(w)
    rb = L.router() if router_bits is None else router_bits
    router = torch.from_numpy(rb.view(np.int16)).view(torch.bfloat16).cuda()
    dummy = torch.zeros(256, dtype=torch.uint8, device="cuda")
    lay = bm.Layer(w.H, w.I, w.E, w.k, router, dummy, dummy, dummy, dummy)
    logits = torch.empty((x.shape[0], w.E), dtype=torch.float32, device="cuda")
    ids, wt = bm.route(lay, x_to_device(x), logits=logits)
    torch.cuda.synchronize()
    return ids.cpu().numpy(), wt.cpu().numpy(), logits.cpu().numpy()


def _check_route(w, x, router_bits=None):
    L = synth_layer(w)
    rb = L.router() if router_bits is None else router_bits
    ref_logits = oracle.router_logits(x, rb)
    rid, rw = oracle.topk(ref_logits, w.k)
    gid, gw, glog = _route_gpu(w, x, router_bits)
    # logits: fp32 accumulation of exact products
    scale = np.abs(ref_logits).max()
    np.testing.assert_allclose(glog, ref_logits, rtol=0, atol=2e-5 * max(scale, 1.0))
    ties = set(near_tie_tokens(ref_logits, w.k).tolist())
    ok = np.array([t not in ties for t in range(x.shape[0])])
    say(f"[route] {w.name} T={x.shape[0]} near-ties={len(ties)} "
        f"max|dlogit|={float(np.abs(glog - ref_logits).max()):.2e}")
    np.testing.assert_array_equal(gid[ok], rid[ok])
    # w_j = exp(l_j - l_1) / sum_i exp(l_i - l_1): a logit error d moves each
    # weight by at most w_j * 2 max|d| <= 2 max|d| (+ fp32 exp/divide rounding)
    dl = float(np.abs(glog - ref_logits).max())
    np.testing.assert_allclose(gw[ok], rw[ok], rtol=0, atol=2 * dl + 1e-6)
    np.testing.assert_allclose(gw.sum(axis=1), 1.0, atol=1e-6)
    for t in ties:          # several answers are correct: check validity
        kth = -np.sort(-ref_logits[t])[w.k - 1]
        assert len(set(gid[t].tolist())) == w.k
        assert np.all(ref_logits[t, gid[t]] >= kth - 1e-4)


def test_route_tiny_fp32():
    require_gpu()
    w = synth.WORKLOADS["tiny"]
    x, _ = synth.make_tokens(w)
    _check_route(w, x)


def test_route_decode_b1():
    require_gpu()
    w = synth.WORKLOADS["decode_b1"]
    x, _ = synth.make_tokens(w)
    _check_route(w, x)


def test_route_batch16_bf16_and_fp32():
    """16 tokens: two token batches of the split-K router, both dtypes."""
    require_gpu()
    w = synth.WORKLOADS["decode_b1"].with_(T=16)
    x, _ = synth.make_tokens(w)
    _check_route(w, x)
    xf = synth.f32_from_bf16_bits(x) + np.float32(1e-3)   # fp32 values off the bf16 grid
    _check_route(w.with_(x_dtype="f32"), xf.astype(np.float32))


def test_route_prefill_mfma_path():
    """2048 bf16 tokens go through the MFMA router GEMM."""
    require_gpu()
    w = synth.WORKLOADS["prefill_2k"]
    x, _ = synth.make_tokens(w)
    _check_route(w, x)


def test_route_ragged_and_small_expert_counts():
    require_gpu()
    for E, k, T in ((33, 5, 70), (5, 5, 3), (8, 1, 65), (100, 16, 9)):
        w = synth.Workload(f"r{E}_{k}", T, 512, 256, E, k, "bf16", "computed", None, False, 11, "decode")
        x, _ = synth.make_tokens(w)
        _check_route(w, x)


def test_route_mfma_odd_stage_slices():
    """The matrix-core router's K slices with an odd number of 64-wide stages
    and a short last slice (H 2304: seven slices of 5 stages, one of 1),
    tokens past the last 64-token tile and experts past the last full tile."""
    require_gpu()
    w = synth.Workload("r_odd", 130, 2304, 256, 200, 6, "bf16", "computed", None, False, 13, "decode")
    x, _ = synth.make_tokens(w)
    _check_route(w, x)


def test_route_zero_input_ties_to_lowest_index():
    require_gpu()
    w = synth.WORKLOADS["decode_b1"].with_(T=3)
    x = np.zeros((3, w.H), dtype=np.uint16)
    gid, gw, _ = _route_gpu(w, x)
    assert gid.tolist() == [list(range(w.k))] * 3
    np.testing.assert_allclose(gw, 1.0 / w.k, atol=1e-7)


@pytest.mark.parametrize("name", ["decode_b16_zipf", "prefill_8k_zipf"])
def test_topk_on_drawn_logits(name):
    """Both sides select from the same fp32 logits: ids must match exactly."""
    require_gpu()
    import bit_moe_amd as bm
    w = synth.WORKLOADS[name]
    lg = synth.zipf_logits(w)
    rid, rw = oracle.topk(lg.astype(np.float64), w.k)
    gid, gw = bm.topk(torch.from_numpy(lg).cuda(), w.k)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(gid.cpu().numpy(), rid)
    np.testing.assert_allclose(gw.cpu().numpy(), rw, atol=1e-6)


@pytest.mark.parametrize("E,k", [(200, 8), (256, 16), (1000, 6)])
def test_topk_signed_zero_ties_and_expert_counts(E, k):
    """Random logits with planted exact ties, including -0.0 against +0.0
    (equal values: the lower expert index wins), for expert counts below,
    at and above one wave's four logits per lane."""
    require_gpu()
    import bit_moe_amd as bm
    rng = np.random.default_rng(E + k)
    lg = rng.standard_normal((24, E)).astype(np.float32)
    lg[:, 5] = lg[:, 3]                       # exact ties
    lg[0, :] = 0.0
    lg[0, 1::2] = -0.0                       # signed zeros only: experts 0..k-1
    lg[1, : E // 2] = -0.0
    lg[1, E // 2:] = -1.0                    # -0.0 wins, lowest indices first
    rid, rw = oracle.topk(lg.astype(np.float64), k)
    gid, gw = bm.topk(torch.from_numpy(lg).cuda(), k)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(gid.cpu().numpy(), rid)
    np.testing.assert_allclose(gw.cpu().numpy(), rw, atol=1e-6)
    assert gid.cpu().numpy()[0].tolist() == list(range(k))


def _bucket_case(ids, E):
    import bit_moe_amd as bm
    counts, offsets, perm = oracle.bucket(ids, E)
    g = bm.bucket(torch.from_numpy(ids).cuda(), E)
    torch.cuda.synchronize()
    gc, go, gp, ga, gn = (t.cpu().numpy() for t in g)
    np.testing.assert_array_equal(gc, counts)
    np.testing.assert_array_equal(go, offsets)
    np.testing.assert_array_equal(gp, perm)
    act = np.nonzero(counts)[0]
    assert gn[0] == len(act)
    np.testing.assert_array_equal(ga[:len(act)], act)
    assert np.all(ga[len(act):] == -1)


@pytest.mark.parametrize("T,k,E,skew", [
    (1, 8, 256, 0), (4, 2, 8, 0), (16, 8, 256, 1.1), (600, 8, 256, 0),       # single-block path
    (2048, 8, 256, 0), (8192, 8, 256, 1.2), (777, 3, 1000, 0),              # multi-block path
    (5000, 16, 1024, 0.8), (1, 1, 1, 0),
])
def test_bucket_exact(T, k, E, skew):
    require_gpu()
    say(f"[bucket] T={T} k={k} E={E} skew={skew}")
    if skew:
        w = synth.Workload("b", T, 256, 256, E, k, "bf16", "zipf", skew, False, 5, "prefill")
        ids, _ = oracle.topk(synth.zipf_logits(w).astype(np.float64), k)
    else:
        rng = np.random.default_rng(T * 31 + E)
        ids = np.argsort(rng.random((T, E)), axis=1)[:, :k].astype(np.int32)
    _bucket_case(ids, E)


def test_bucket_all_tokens_one_expert_set():
    require_gpu()
    ids = np.tile(np.array([7, 3, 250], dtype=np.int32), (3000, 1))
    _bucket_case(ids, 256)
