"""GPU parity: the MoE FFN (decode and prefill entry points) against the
oracle, max|err| <= 2e-2 * rms(oracle output) with fp32 accumulation.

The FFN tests feed both sides the same ids and weights (the oracle's
routing, as float32), so the FFN is checked on its own; an end-to-end test
routes on the GPU as well.  Full-size prefill chunks are compared on a
sample of tokens the oracle computes one by one (hottest and coldest
experts included)."""
import numpy as np
import pytest

import oracle
import synth
from _gpu import (W_TOL, assert_close_rms, device_layer, near_tie_tokens, require_gpu, say, synth_layer,
                  torch, x_to_device)

pytestmark = pytest.mark.gpu


def _routing(w, x):
    """ids int32 [T,k] and weights as float32 (what the GPU receives)."""
    L = synth_layer(w)
    if w.routing == "zipf":
        ids, wt = oracle.topk(synth.zipf_logits(w, T=x.shape[0]).astype(np.float64), w.k)
    else:
        ids, wt = oracle.route(x, L.router(), w.k)
    return ids.astype(np.int32), wt.astype(np.float32)


def _gpu_ffn(w, x, ids, wt, mode):
    import bit_moe_amd as bm
    lay = device_layer(w)
    fn = bm.ffn_decode if mode == "decode" else bm.ffn_prefill
    y = fn(lay, x_to_device(x), torch.from_numpy(ids).cuda(), torch.from_numpy(wt).cuda())
    torch.cuda.synchronize()
    return y.cpu().numpy()


def _oracle_rows(w, x, ids, wt, rows):
    L = synth_layer(w)
    return oracle.layer_ffn(L, x[rows], ids[rows], wt[rows].astype(np.float64))


@pytest.mark.parametrize("mode", ["decode", "prefill"])
def test_tiny_layer_all_tokens(mode):
    require_gpu()
    w = synth.WORKLOADS["tiny"]
    x, _ = synth.make_tokens(w)
    ids, wt = _routing(w, x)
    y = _gpu_ffn(w, x, ids, wt, mode)
    ref = _oracle_rows(w, x, ids, wt, np.arange(w.T))
    assert_close_rms(y, ref, what=f"tiny/{mode}")


@pytest.mark.parametrize("mode", ["decode", "prefill"])
def test_tiny_shapes_with_shared_and_ragged_tokens(mode):
    """Shared expert present, T not a multiple of any tile, bf16 and fp32."""
    require_gpu()
    for xd, T in (("bf16", 37), ("f32", 5)):
        w = synth.WORKLOADS["tiny"].with_(name=f"tiny_sh_{xd}", T=T, shared=True, x_dtype=xd, seed=21)
        x, _ = synth.make_tokens(w)
        ids, wt = _routing(w, x)
        y = _gpu_ffn(w, x, ids, wt, mode)
        ref = _oracle_rows(w, x, ids, wt, np.arange(T))
        assert_close_rms(y, ref, what=f"tiny-shared/{xd}/{mode}/T={T}")


@pytest.mark.parametrize("T", [2, 3])
def test_tiny_decode_few_tokens_shared_both_dtypes(T):
    """2 or 3 tokens with a shared expert (one gate/up and one down launch
    for every expert, the shared gate/up partial sums from the front launch),
    bf16 and fp32 activations."""
    require_gpu()
    for xd in ("bf16", "f32"):
        w = synth.WORKLOADS["tiny"].with_(name=f"tiny_few_{xd}", T=T, shared=True, x_dtype=xd, seed=70 + T)
        x, _ = synth.make_tokens(w)
        ids, wt = _routing(w, x)
        ref = _oracle_rows(w, x, ids, wt, np.arange(T))
        assert_close_rms(_gpu_ffn(w, x, ids, wt, "decode"), ref, what=f"tiny few tokens/{xd}/T={T}")


def test_decode_b1_full():
    require_gpu()
    w = synth.WORKLOADS["decode_b1"]
    x, _ = synth.make_tokens(w)
    ids, wt = _routing(w, x)
    say(f"[ffn] decode_b1 ids={ids.tolist()}")
    y = _gpu_ffn(w, x, ids, wt, "decode")
    ref = _oracle_rows(w, x, ids, wt, np.arange(1))
    assert_close_rms(y, ref, what="decode_b1")


def test_decode_b16_zipf_full():
    require_gpu()
    w = synth.WORKLOADS["decode_b16_zipf"]
    x, _ = synth.make_tokens(w)
    ids, wt = _routing(w, x)
    say(f"[ffn] decode_b16_zipf distinct experts={len(np.unique(ids))}")
    y = _gpu_ffn(w, x, ids, wt, "decode")
    ref = _oracle_rows(w, x, ids, wt, np.arange(w.T))
    assert_close_rms(y, ref, what="decode_b16_zipf")


@pytest.mark.parametrize("k", [1, 3, 4, 16])
def test_decode_one_token_shared_every_k(k):
    """One token with a shared expert.  k a power of two: the k gate/up
    workgroups of each panel also take 64/k of its shared rows each over all
    of K (k = 1: all 64 rows; k = 16: four), on four waves that deal out the
    160 (H 1280) or 96 (H 768) pieces of a row in rounds of 4 * k pieces:
    a ragged last round at k = 16 (64 per round); at k = 4 (16 per round)
    6 or 10 rounds, fewer and more than run before the routing barrier.
    k = 3: the front launch's K chunks.  bf16 and fp32 activations, both
    entry points that take one token (given ids, and routing on the GPU)."""
    require_gpu()
    import bit_moe_amd as bm
    for xd, H in (("bf16", 1280), ("f32", 768)):
        w = synth.WORKLOADS["tiny"].with_(name=f"tiny_sr{k}_{xd}", T=1, H=H, E=32, k=k, shared=True, x_dtype=xd,
                                          seed=60 + k)
        L = synth_layer(w)
        x, _ = synth.make_tokens(w, accept=lambda t, r: oracle.margin_ok(r, L.router(), w.k, 1e-4))
        ids, wt = _routing(w, x)
        ref = _oracle_rows(w, x, ids, wt, np.arange(1))
        assert_close_rms(_gpu_ffn(w, x, ids, wt, "decode"), ref, what=f"one token k={k} {xd} H={H}")
        y, gid, gw = bm.forward_decode(device_layer(w), x_to_device(x))
        torch.cuda.synchronize()
        np.testing.assert_array_equal(gid.cpu().numpy(), ids)
        assert_close_rms(y.cpu().numpy(), ref, what=f"one token routed on the GPU k={k} {xd} H={H}")


PF_TILE_ROWS = 96      # rows per prefill row tile (blocks of 32 rows)


def _sample_rows(ids, E, n_random, seed):
    """Tokens whose rows cover the prefill tile classes: one row from every
    row tile of the hottest and the coldest expert (first rows, and the last
    row of the expert), the last row of partial tails holding 1-32, 33-64
    and 65-96 rows (one, two and three 32-row blocks) for two experts each,
    plus n_random random tokens.  Row r of expert e is bucket slot
    offsets[e] + r (the oracle's bucketing), pair perm[slot], token pair // k."""
    rng = np.random.default_rng(seed)
    T, k = ids.shape
    counts, offsets, perm = oracle.bucket(ids, E)
    tok_of = lambda e, r: int(perm[offsets[e] + r]) // k
    used = np.nonzero(counts)[0]
    hot = int(used[np.argmax(counts[used])])
    cold = int(used[np.argmin(counts[used])])
    rows = set()
    for e in (hot, cold):
        c = int(counts[e])
        rows |= {tok_of(e, r0) for r0 in range(0, c, PF_TILE_ROWS)}
        rows.add(tok_of(e, c - 1))
    classes = {1: [], 2: [], 3: []}
    for e in used:
        tail = int(counts[e]) % PF_TILE_ROWS or PF_TILE_ROWS
        classes[(tail + 31) // 32].append(int(e))
    for mb, es in classes.items():
        for e in es[:2]:
            c = int(counts[e])
            rows |= {tok_of(e, c - 1), tok_of(e, (c - 1) // PF_TILE_ROWS * PF_TILE_ROWS)}
    rows |= set(rng.choice(T, size=n_random, replace=False).tolist()) | {0, T - 1}
    say(f"[sample] hot e{hot} ({counts[hot]} rows, {(counts[hot] + PF_TILE_ROWS - 1) // PF_TILE_ROWS} tiles), "
        f"cold e{cold} ({counts[cold]} rows), tail classes "
        f"{ {mb: len(es) for mb, es in classes.items()} }, {len(rows)} tokens")
    return np.array(sorted(rows))


@pytest.mark.parametrize("name", ["prefill_2k", "prefill_8k_zipf"])
def test_prefill_full_size_sampled(name):
    """Full-size prefill chunks at the launch configuration the bench times,
    compared on at least 64 tokens the oracle computes one by one, chosen
    to reach every row tile of the hottest and coldest expert and every
    tile size class."""
    require_gpu()
    w = synth.WORKLOADS[name]
    x, _ = synth.make_tokens(w)
    ids, wt = _routing(w, x)
    c = np.bincount(ids.ravel(), minlength=w.E)
    say(f"[ffn] {name} rows/expert max={c.max()} min={c.min()} active={np.count_nonzero(c)}")
    y = _gpu_ffn(w, x, ids, wt, "prefill")
    rows = _sample_rows(ids, w.E, 56, 1)
    assert len(rows) >= 64
    ref = _oracle_rows(w, x, ids, wt, rows)
    assert_close_rms(y[rows], ref, what=f"{name} {len(rows)} sampled tokens")
    assert np.all(np.isfinite(y))


def test_decode_and_prefill_agree_and_batch_rows_match_single_tokens():
    require_gpu()
    w = synth.WORKLOADS["decode_b16_zipf"]
    x, _ = synth.make_tokens(w)
    ids, wt = _routing(w, x)
    yd = _gpu_ffn(w, x, ids, wt, "decode")
    yp = _gpu_ffn(w, x, ids, wt, "prefill")
    assert_close_rms(yp, yd.astype(np.float64), what="prefill vs decode")
    # a token alone runs every expert on the single-token kernels; in the
    # batch, experts chosen by several tokens take the matrix-core kernels,
    # so rows agree to the FFN tolerance, not bit for bit
    for t in (0, 7, 15):
        y1 = _gpu_ffn(w, x[t:t + 1], ids[t:t + 1], wt[t:t + 1], "decode")
        assert_close_rms(yd[t:t + 1], y1.astype(np.float64), what=f"batch row {t} vs alone")


def test_deterministic_repeat():
    require_gpu()
    w = synth.WORKLOADS["decode_b16_zipf"]
    x, _ = synth.make_tokens(w)
    ids, wt = _routing(w, x)
    for mode in ("decode", "prefill"):
        a = _gpu_ffn(w, x, ids, wt, mode)
        b = _gpu_ffn(w, x, ids, wt, mode)
        np.testing.assert_array_equal(a, b)


def test_zero_activation_gives_zero():
    require_gpu()
    w = synth.WORKLOADS["decode_b16_zipf"]
    x = np.zeros((4, w.H), dtype=np.uint16)
    ids = np.array([[0, 1, 2, 3, 4, 5, 6, 7]] * 4, dtype=np.int32)
    wt = np.full((4, 8), 0.125, dtype=np.float32)
    for mode in ("decode", "prefill"):
        assert np.all(_gpu_ffn(w, x, ids, wt, mode) == 0.0)


def test_hot_expert_many_tiles_and_unused_experts():
    """Every token picks the same k experts: one expert bucket spans many
    row tiles, all other experts are empty."""
    require_gpu()
    w = synth.WORKLOADS["tiny"].with_(name="tiny_hot", T=300, x_dtype="bf16", seed=5)
    x, _ = synth.make_tokens(w)
    ids = np.tile(np.array([6, 1], dtype=np.int32), (w.T, 1))
    wt = np.tile(np.array([0.7, 0.3], dtype=np.float32), (w.T, 1))
    ref = _oracle_rows(w, x, ids, wt, np.arange(w.T))
    for mode in ("decode", "prefill"):
        assert_close_rms(_gpu_ffn(w, x, ids, wt, mode), ref, what=f"hot/{mode}")


def test_single_expert_single_slot():
    require_gpu()
    w = synth.WORKLOADS["tiny"].with_(name="tiny_k1", k=1, T=3, seed=8)
    x, _ = synth.make_tokens(w)
    ids = np.array([[3], [3], [0]], dtype=np.int32)
    wt = np.ones((3, 1), dtype=np.float32)
    ref = _oracle_rows(w, x, ids, wt, np.arange(3))
    for mode in ("decode", "prefill"):
        assert_close_rms(_gpu_ffn(w, x, ids, wt, mode), ref, what=f"k1/{mode}")


def test_end_to_end_route_then_ffn():
    require_gpu()
    import bit_moe_amd as bm
    w = synth.WORKLOADS["decode_b1"].with_(T=4, name="decode_b4")
    x, _ = synth.make_tokens(w)
    lay = device_layer(synth.WORKLOADS["decode_b1"])
    L = synth_layer(synth.WORKLOADS["decode_b1"])
    xd = x_to_device(x)
    gid, gw = bm.route(lay, xd)
    y = bm.ffn_decode(lay, xd, gid, gw)
    torch.cuda.synchronize()
    lg = oracle.router_logits(x, L.router())
    assert len(near_tie_tokens(lg, w.k)) == 0
    rid, rw = oracle.topk(lg, w.k)
    np.testing.assert_array_equal(gid.cpu().numpy(), rid)
    ref = oracle.layer_ffn(L, x, rid, rw)
    assert_close_rms(y.cpu().numpy(), ref, what="route+decode")


@pytest.mark.parametrize("T", [1, 2, 3, 4, 8, 9, 16, 20, 64, 200])
def test_forward_decode_routes_and_matches_oracle(T):
    """moe_forward_decode (router fused into the first launch for T <= 16,
    separate routing above: the one-wave-per-row router below 64 bf16
    tokens, the split-K matrix-core router from 64) against oracle routing
    + FFN.  2 to 8 tokens take one decode launch for all experts, 9 to 96
    the prefill kernels beside them for experts chosen by several tokens."""
    require_gpu()
    import bit_moe_amd as bm
    w0 = synth.WORKLOADS["decode_b1"]
    w = w0.with_(T=T, name=f"fwd{T}")
    L = synth_layer(w0)
    x, _ = synth.make_tokens(w, accept=lambda t, r: oracle.margin_ok(r, L.router(), w.k, 1e-4))
    lay = device_layer(w0)
    y, gid, gw = bm.forward_decode(lay, x_to_device(x))
    torch.cuda.synchronize()
    rid, rw = oracle.route(x, L.router(), w.k)
    np.testing.assert_array_equal(gid.cpu().numpy(), rid)
    np.testing.assert_allclose(gw.cpu().numpy(), rw, atol=W_TOL)
    ref = oracle.layer_ffn(L, x, rid, rw)
    assert_close_rms(y.cpu().numpy(), ref, what=f"forward_decode T={T}")


@pytest.mark.parametrize("T", [1, 3])
def test_forward_decode_small_expert_count(T):
    """E = 8 experts (fewer than a wave's lanes: the in-launch top-k sees
    missing entries), shared expert, bf16: GPU routing + FFN against the
    oracle's."""
    require_gpu()
    import bit_moe_amd as bm
    w = synth.WORKLOADS["tiny"].with_(name=f"tiny_fwd{T}", T=T, shared=True, x_dtype="bf16", seed=31)
    L = synth_layer(w)
    x, _ = synth.make_tokens(w, accept=lambda t, r: oracle.margin_ok(r, L.router(), w.k, 1e-4))
    y, gid, gw = bm.forward_decode(device_layer(w), x_to_device(x))
    torch.cuda.synchronize()
    rid, rw = oracle.route(x, L.router(), w.k)
    np.testing.assert_array_equal(gid.cpu().numpy(), rid)
    np.testing.assert_allclose(gw.cpu().numpy(), rw, atol=W_TOL)
    ref = oracle.layer_ffn(L, x, rid, rw)
    assert_close_rms(y.cpu().numpy(), ref, what=f"forward_decode E=8 T={T}")


@pytest.mark.parametrize("T", [2, 6, 13])
def test_forward_decode_router_rows_past_expert_count(T):
    """E = 30 experts: for several tokens the front launch's router rows take
    four waves each, four rows per workgroup, so the last workgroup holds rows
    past E (not written); token counts on the 4-, 8- and 16-token passes."""
    require_gpu()
    import bit_moe_amd as bm
    w = synth.WORKLOADS["tiny"].with_(name=f"tiny_e30_{T}", T=T, E=30, k=6, shared=True, x_dtype="bf16", seed=37)
    L = synth_layer(w)
    x, _ = synth.make_tokens(w, accept=lambda t, r: oracle.margin_ok(r, L.router(), w.k, 1e-4))
    y, gid, gw = bm.forward_decode(device_layer(w), x_to_device(x))
    torch.cuda.synchronize()
    rid, rw = oracle.route(x, L.router(), w.k)
    np.testing.assert_array_equal(gid.cpu().numpy(), rid)
    np.testing.assert_allclose(gw.cpu().numpy(), rw, atol=W_TOL)
    ref = oracle.layer_ffn(L, x, rid, rw)
    assert_close_rms(y.cpu().numpy(), ref, what=f"forward_decode E=30 T={T}")


@pytest.mark.parametrize("copies", [4, 12])
@pytest.mark.parametrize("shared", [False, True])
def test_forward_decode_all_experts_shared_by_tokens(shared, copies):
    """Copies of one token: every chosen expert has one pair per copy.  Twelve
    copies: the batch's experts all go through the matrix-core kernels and,
    without a shared expert, no single-token expert is left to combine the
    outputs; four copies: the one decode launch for all experts, every item
    a pass of four tokens."""
    require_gpu()
    import bit_moe_amd as bm
    w = synth.WORKLOADS["tiny"].with_(name=f"tiny_rep_{int(shared)}", T=1, shared=shared, x_dtype="bf16", seed=41)
    L = synth_layer(w)
    x1, _ = synth.make_tokens(w, accept=lambda t, r: oracle.margin_ok(r, L.router(), w.k, 1e-4))
    x = np.repeat(x1, copies, axis=0)
    y, gid, gw = bm.forward_decode(device_layer(w), x_to_device(x))
    torch.cuda.synchronize()
    rid, rw = oracle.route(x, L.router(), w.k)
    np.testing.assert_array_equal(gid.cpu().numpy(), rid)
    np.testing.assert_allclose(gw.cpu().numpy(), rw, atol=W_TOL)
    ref = oracle.layer_ffn(L, x, rid, rw)
    assert_close_rms(y.cpu().numpy(), ref, what=f"forward_decode {copies} equal tokens shared={shared}")


@pytest.mark.parametrize("T", [1, 4])
def test_forward_decode_zero_input_ties(T):
    """x = 0: every logit ties, so the top-k is experts 0..k-1 with weight
    1/k each (lowest index first), and y = 0 exactly."""
    require_gpu()
    import bit_moe_amd as bm
    w = synth.WORKLOADS["decode_b1"]
    x = np.zeros((T, w.H), dtype=np.uint16)
    y, gid, gw = bm.forward_decode(device_layer(w), x_to_device(x))
    torch.cuda.synchronize()
    assert gid.cpu().numpy().tolist() == [list(range(w.k))] * T
    np.testing.assert_allclose(gw.cpu().numpy(), 1.0 / w.k, atol=1e-7)
    assert not np.any(y.cpu().numpy())


def _scaled_layer_case(w, d_of_block):
    """The tiny layer's canonical blocks with every superblock scale (IQ2X d;
    Q2K d and dmin) replaced by d_of_block(n) (fp16 values), uploaded and
    packed; returns (device layer, gate, up, down per expert)."""
    import bit_moe_amd as bm
    L = synth_layer(w)
    gate, up, down = L.gate_all().copy(), L.up_all().copy(), L.down_all().copy()
    for arr, cols in ((gate, [(0, 2)]), (up, [(0, 2)]), (down, [(80, 82), (82, 84)])):
        for a, b in cols:
            d = d_of_block(arr.shape[0]).astype(np.float16)
            arr[:, a:b] = d.view(np.uint8).reshape(-1, 2)
    lay = bm.layer_from_canonical(w.H, w.I, w.E, w.k, L.router(), gate, up, down, L.grid(), None)
    ng, nd = w.I * (w.H // 256), w.H * (w.I // 256)
    per = lambda a, n: {e: a[e * n:(e + 1) * n] for e in range(w.E)}
    return lay, per(gate, ng), per(up, ng), per(down, nd)


@pytest.mark.parametrize("case", ["d=8", "d=2^-19", "per-expert log-uniform"])
def test_scale_envelope_both_paths(case):
    """Superblock scales at both ends of the range the prefill fp16 operands
    hold exactly in their normal range (d, dmin in [2^-19, 8]: largest IQ2X
    weight 27.1 d, largest Q2K term 45 d), and one scale per expert tensor
    drawn log-uniformly over it (experts 2^22 apart in one token's sum);
    decode and prefill against the oracle on the same blocks."""
    require_gpu()
    w = synth.WORKLOADS["tiny"].with_(name=f"tiny_env", T=37, x_dtype="bf16", seed=51)
    rng = np.random.default_rng(5)

    def per_expert(n):
        per = n // w.E
        return np.repeat(np.exp2(rng.uniform(-19, 3, w.E)), per)
    pick = {"d=8": lambda n: np.full(n, 8.0),
            "d=2^-19": lambda n: np.full(n, 2.0 ** -19),
            "per-expert log-uniform": per_expert}[case]
    lay, gate, up, down = _scaled_layer_case(w, pick)
    x, _ = synth.make_tokens(w)
    ids, wt = _routing(w, x)
    L = synth_layer(w)
    ref = oracle.moe_ffn(w.H, w.I, w.E, w.k, L.grid(), gate, up, down, None, x, ids, wt.astype(np.float64))
    assert np.all(np.isfinite(ref))
    import bit_moe_amd as bm
    for mode, fn in (("decode", bm.ffn_decode), ("prefill", bm.ffn_prefill)):
        y = fn(lay, x_to_device(x), torch.from_numpy(ids).cuda(), torch.from_numpy(wt).cuda())
        torch.cuda.synchronize()
        assert_close_rms(y.cpu().numpy(), ref, what=f"scale envelope {case}/{mode}")
