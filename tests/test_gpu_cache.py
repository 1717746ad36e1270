"""GPU: the routed-expert residency cache (moe_cache_*).  The experts' tiled
slabs sit in pinned host memory and a pool of HBM slots holds the ones in
use; each step maps its routing onto slots (copying missing experts in on
the stream) and runs the decode FFN on the pool.  The same kernels read the
same bytes, so every step's output must equal, bit for bit, the output of
the fully resident layer with the original ids; one step is also checked
against the oracle, and the slot sequence against the LRU model."""
import numpy as np
import pytest

import oracle
import synth
from _gpu import assert_close_rms, device_layer, require_gpu, say, synth_layer, torch, x_to_device
from test_sanitizers import _lru_model

pytestmark = pytest.mark.gpu


def _cache_for(w, slots):
    import bit_moe_amd as bm
    lay = device_layer(w)
    host = tuple(t.cpu().pin_memory() for t in lay.tensors[1:4])    # tiled gate, up, down of all experts
    return lay, bm.ExpertCache(lay, host, slots)


def _run(w, slots, steps, routing):
    """steps x routing: yields (y_cache, y_resident, ids, x, loaded) per step."""
    import bit_moe_amd as bm
    lay, cache = _cache_for(w, slots)
    out = []
    for i in range(steps):
        wi = w.with_(seed=w.seed + 1000 + i)
        x, _ = synth.make_tokens(wi)
        xd = x_to_device(x)
        if routing == "zipf":
            ids_d, wt = bm.topk(torch.from_numpy(synth.zipf_logits(wi)).cuda(), w.k)
        else:
            ids_d, wt = bm.route(lay, xd)
        ids_h = ids_d.cpu()
        slot_h, loaded = cache.map(ids_h)
        yc = bm.ffn_decode(cache.layer, xd, slot_h.cuda(), wt)
        yr = bm.ffn_decode(lay, xd, ids_d, wt)
        torch.cuda.synchronize()
        out.append((yc.cpu().numpy(), yr.cpu().numpy(), ids_h.numpy(), x, wt.cpu().numpy(), loaded))
    hits, misses, _ = cache.stats()
    cache.close()
    return out, hits, misses


def test_tiny_layer_cache_steps_match_resident_and_lru_model():
    require_gpu()
    w = synth.WORKLOADS["tiny"].with_(name="tiny_cache", T=3, shared=True, x_dtype="bf16", seed=71)
    # 6 slots of 8 experts: a step (3 tokens, top-2) needs at most 6
    out, hits, misses = _run(w, 6, 12, "computed")
    model = _lru_model([list(o[2].ravel()) for o in out], w.E, 6)
    for i, (yc, yr, ids, x, wt, loaded) in enumerate(out):
        np.testing.assert_array_equal(yc, yr)
        assert loaded == model[i][1], (i, loaded, model[i])
    assert (hits, misses) == model[-1][3:]
    yc, _, ids, x, wt, _ = out[-1]
    ref = oracle.layer_ffn(synth_layer(w), x, ids, wt.astype(np.float64))
    assert_close_rms(yc, ref, what="cache step vs oracle")
    say(f"[cache] tiny: hits {hits} misses {misses}")


@pytest.mark.parametrize("name,slots,steps", [("decode_b1", 24, 6), ("decode_b16_zipf", 96, 4)])
def test_full_shape_cache_steps_match_resident(name, slots, steps):
    """H 7168, I 2048, 256 experts: one token per step (24 slots, so the
    cache evicts from the fourth step), and 16-token Zipf(1.1) batches (96
    slots; experts chosen by several tokens take the matrix-core kernels)."""
    require_gpu()
    w = synth.WORKLOADS[name]
    out, hits, misses = _run(w, slots, steps, "zipf" if w.routing == "zipf" else "computed")
    for i, (yc, yr, ids, x, wt, loaded) in enumerate(out):
        say(f"[cache] {name} step {i}: {loaded} experts copied")
        np.testing.assert_array_equal(yc, yr)
    assert misses > 0 and hits + misses == sum(len(np.unique(o[2])) for o in out)


def test_mxfp4_layer_cache_steps_match_resident():
    """The cache over an MXFP4 layer (slabs of 17 bytes per 32 weights): every
    step equals the resident layer bit for bit, the copies follow the LRU
    model, and one step matches the oracle."""
    require_gpu()
    w = synth.WORKLOADS["tiny"].with_(name="tiny_cache_mx", T=3, shared=True, x_dtype="bf16", seed=73,
                                      fmt="mxfp4")
    out, hits, misses = _run(w, 6, 10, "computed")
    model = _lru_model([list(o[2].ravel()) for o in out], w.E, 6)
    for i, (yc, yr, ids, x, wt, loaded) in enumerate(out):
        np.testing.assert_array_equal(yc, yr)
        assert loaded == model[i][1], (i, loaded, model[i])
    assert (hits, misses) == model[-1][3:]
    yc, _, ids, x, wt, _ = out[-1]
    ref = oracle.layer_ffn(synth_layer(w), x, ids, wt.astype(np.float64))
    assert_close_rms(yc, ref, what="mxfp4 cache step vs oracle")
