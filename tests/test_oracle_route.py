"""Pins of the oracle's routing and bucketing (CPU only).

Routing: the router picks a few experts per token (page "Un modele de 284
milliards de parametres tourne desormais sur un Mac de 128 Go. Qui y perd ?",
section "Comment un modele de 284 milliards de parametres tient sur une seule
machine"); the layer keeps the k largest logits and renormalises their
softmax.  The oracle takes the softmax over the selected k only; the brute
force below takes the full softmax over all E experts and renormalises, which
must agree because the shared denominator cancels.
"""
import numpy as np
import pytest

import oracle
import synth


def _bf16_as_f64(bits):
    return synth.f32_from_bf16_bits(bits).astype(np.float64)


def _brute_route(logits, k):
    T, E = logits.shape
    ids = np.empty((T, k), dtype=np.int32)
    w = np.empty((T, k))
    for t in range(T):
        l = logits[t]
        p = np.exp(l - l.max())
        p /= p.sum()                                  # full softmax over E
        order = np.lexsort((np.arange(E), -l))        # logit desc, index asc
        sel = order[:k]
        ids[t] = sel
        w[t] = p[sel] / p[sel].sum()                  # renormalise over the k
    return ids, w


def test_router_logits_match_float64_matmul():
    w = synth.WORKLOADS["tiny"]
    L = synth.make_layer(w)
    x, _ = synth.make_tokens(w)
    got = oracle.router_logits(x, L.router())
    ref = x.astype(np.float64) @ _bf16_as_f64(L.router()).T
    np.testing.assert_allclose(got, ref, rtol=1e-12, atol=1e-12)
    # bf16 activations take the same path
    xb = synth.bf16_bits_from_f32(x)
    got_b = oracle.router_logits(xb, L.router())
    ref_b = _bf16_as_f64(xb) @ _bf16_as_f64(L.router()).T
    np.testing.assert_allclose(got_b, ref_b, rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("T,E,k", [(7, 8, 2), (5, 256, 8), (3, 33, 16), (4, 5, 5), (2, 9, 1)])
def test_topk_matches_full_softmax_brute_force(T, E, k):
    rng = np.random.default_rng(T * 1000 + E)
    logits = rng.standard_normal((T, E))
    ids, w = oracle.topk(logits, k)
    bi, bw = _brute_route(logits, k)
    np.testing.assert_array_equal(ids, bi)
    np.testing.assert_allclose(w, bw, rtol=1e-12, atol=1e-15)
    np.testing.assert_allclose(w.sum(axis=1), 1.0, rtol=0, atol=1e-14)
    assert np.all(np.diff(w, axis=1) <= 0)
    for t in range(T):
        assert len(set(ids[t].tolist())) == k


def test_topk_ties_go_to_lower_index():
    logits = np.array([[0.5, 1.0, 1.0, 0.2, 1.0, 0.5]])
    ids, w = oracle.topk(logits, 4)
    assert ids.tolist() == [[1, 2, 4, 0]]
    np.testing.assert_allclose(w[0, :3], w[0, 0])


def test_zero_activation_routes_to_first_k_evenly():
    w = synth.WORKLOADS["tiny"]
    L = synth.make_layer(w)
    x = np.zeros((3, w.H), dtype=np.float32)
    ids, wt = oracle.route(x, L.router(), w.k)
    assert ids.tolist() == [list(range(w.k))] * 3
    np.testing.assert_array_equal(wt, np.full((3, w.k), 1.0 / w.k))


def test_single_slot_weight_is_one():
    rng = np.random.default_rng(1)
    l = rng.standard_normal((6, 40))
    ids, w = oracle.topk(l, 1)
    np.testing.assert_array_equal(w, 1.0)
    np.testing.assert_array_equal(ids[:, 0], np.argmax(l, axis=1))


def test_topk_closed_form_two_experts():
    """k=2 weights are the logistic of the logit gap."""
    l = np.array([[0.0, 3.0, -1.0, 1.0]])
    ids, w = oracle.topk(l, 2)
    assert ids.tolist() == [[1, 3]]
    g = 3.0 - 1.0
    np.testing.assert_allclose(w[0], [1 / (1 + np.exp(-g)), 1 / (1 + np.exp(g))], rtol=1e-15)


@pytest.mark.parametrize("T,k,E", [(4, 2, 8), (16, 8, 256), (300, 8, 16), (1, 8, 256), (64, 3, 5)])
def test_bucket_against_library_sort(T, k, E):
    rng = np.random.default_rng(T + k + E)
    ids = np.stack([rng.choice(E, size=k, replace=False) for _ in range(T)]).astype(np.int32)
    counts, offsets, perm = oracle.bucket(ids, E)
    np.testing.assert_array_equal(counts, np.bincount(ids.ravel(), minlength=E))
    np.testing.assert_array_equal(offsets, np.concatenate([[0], np.cumsum(counts)]))
    np.testing.assert_array_equal(perm, np.argsort(ids.ravel(), kind="stable"))
    assert sorted(perm.tolist()) == list(range(T * k))


def test_zipf_logits_skew():
    """The drawn skewed logits make the hottest expert far hotter than the
    coldest (realised histogram is reported in the design notes)."""
    w = synth.WORKLOADS["prefill_8k_zipf"]
    ids, _ = oracle.topk(synth.zipf_logits(w, T=2048), w.k)
    c = np.bincount(ids.ravel(), minlength=w.E)
    assert c.max() > 20 * max(1, np.sort(c)[w.E // 2])
