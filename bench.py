#!/usr/bin/env python3
"""Throughput of the 2-bit routed-expert MoE layer on one MI355X.

One step = one pass of the whole hot path over one batch held in HBM:
moe_forward_decode (router logits, top-k + renormalised softmax, bucketing,
fused IQ2X gate/up dequant-GEMV + SwiGLU, fused Q2K down dequant-GEMV,
gate-weighted combine, bf16 shared expert).

Workload of the headline line: one decode token at DeepSeek-V4-Flash MoE
shapes (H 7168, I 2048, 256 routed experts, top-8, one bf16 shared expert),
seeded synthetic weights.  To keep timed calls out of the 256 MB MALL, the
steps rotate over --copies independent device copies of the layer and over
16 different token rows.  Extra objects report the 16-token Zipf decode
batch and the 2048-token prefill chunk (grouped GEMMs on the fp16 matrix
cores, whose dense peak equals bf16's).

Prints ONE JSON line.
"""
import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK = 8.0e12          # B/s, MI355X HBM3E
BF16_PEAK = 2.5e15         # FLOP/s, dense bf16 (and fp16) MFMA


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--copies", type=int, default=8, help="layer copies rotated to defeat MALL")
    ap.add_argument("--prefill-steps", type=int, default=100, help="timed prefill steps (each workload)")
    ap.add_argument("--prefill-warmup", type=int, default=10)
    ap.add_argument("--cpu-seconds", type=float, default=15.0, help="oracle sample size (seconds)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a plain copy of known size (counter calibration)")
    ap.add_argument("--summarize-kernels", metavar="TRACE_DIR",
                    help="print per-kernel durations of a rocprofv3 --kernel-trace run")
    ap.add_argument("--summarize-traffic", nargs=4, metavar=("FETCH_DIR", "WRITE_DIR", "COPY_FETCH_DIR", "COPY_WRITE_DIR"),
                    help="print the per-kernel HBM traffic summary of four rocprofv3 --pmc runs")
    ap.add_argument("--summarize-mfma", metavar="PMC_DIR",
                    help="print per-kernel MFMA TFLOP/s of a rocprofv3 --pmc SQ_INSTS_VALU_MFMA_MOPS_F16 "
                         "--kernel-trace run")
    ap.add_argument("--summarize-counters", nargs="+", metavar="PMC_DIR",
                    help="print per-kernel averages of every counter of rocprofv3 --pmc runs")
    ap.add_argument("--prefill-only", action="store_true",
                    help="only run the 2048-token prefill step (--prefill-steps times; for counter runs)")
    ap.add_argument("--fmt", choices=("2bit", "mxfp4"), default="2bit",
                    help="routed-expert format of the --prefill-only run")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-extra", action="store_true", help="skip the b16 and prefill lines")
    return ap.parse_args()


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def expert_bytes(w):
    """Bytes of one routed expert's gate+up and down blocks."""
    if w.fmt == "mxfp4":
        return 2 * w.I * (w.H // 32) * 17, w.H * (w.I // 32) * 17
    return 2 * w.I * (w.H // 256) * 66, w.H * (w.I // 256) * 84


def routed_view(bm, w, lay):
    """The layer without its shared expert (the prefill workloads have none)."""
    g = None if lay.fmt == bm.FORMAT_MXFP4 else lay.tensors[4]
    return bm.Layer(w.H, w.I, w.E, w.k, *lay.tensors[:4], g, fmt=lay.fmt)


def build_layer(w, copies):
    import torch
    import bit_moe_amd as bm
    import synth
    L = synth.make_layer(w)
    mx = w.fmt == "mxfp4"
    fmt = bm.FORMAT_MXFP4 if mx else bm.FORMAT_2BIT
    t0 = time.time()
    lay = bm.layer_from_canonical(w.H, w.I, w.E, w.k, L.router(), L.gate_all(), L.up_all(),
                                  L.down_all(), None if mx else L.grid(), L.shared(), fmt=fmt)
    torch.cuda.synchronize()
    log(f"[bench] {w.fmt} layer generated+packed in {time.time() - t0:.1f}s")
    lays = [lay]
    nq = 4 if mx else 5                 # router, gate, up, down (+ grid)
    for _ in range(copies - 1):
        t = [x.clone() for x in lay.tensors]
        sh = tuple(t[nq:nq + 3]) if lay.has_shared else None
        lays.append(bm.Layer(w.H, w.I, w.E, w.k, t[0], t[1], t[2], t[3], None if mx else t[4], sh, fmt=fmt))
    torch.cuda.synchronize()
    return L, lays


def time_steps(step, warmup, steps, dist_steps=None):
    """Run `warmup` untimed steps, then time exactly `steps` steps between a
    synchronize on both sides (one event pair around them: ms per step).
    Then a separate pass of `dist_steps` steps with an event between
    consecutive steps gives the per-step distribution (median, p10, p90;
    each includes one event record, so it reads slightly above the mean of
    the clean pass).  Returns (ms per step, stats)."""
    import torch
    for i in range(warmup):
        step(i)
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for i in range(steps):
        step(warmup + i)
    b.record()
    torch.cuda.synchronize()
    ms = a.elapsed_time(b) / steps
    n = steps if dist_steps is None else dist_steps
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(n + 1)]
    ev[0].record()
    for i in range(n):
        step(warmup + steps + i)
        ev[i + 1].record()
    torch.cuda.synchronize()
    per = sorted(ev[i].elapsed_time(ev[i + 1]) for i in range(n))
    q = lambda f: per[min(len(per) - 1, int(f * (len(per) - 1) + 0.5))]
    stats = {"median_ms": q(0.5), "p10_ms": q(0.1), "p90_ms": q(0.9), "n": n,
             "note": "separate pass, one event record between steps"}
    return ms, stats


def time_kernel(step, n, which):
    """Average duration (ms) of one kernel of the step, from the HIP events
    its dispatch takes at kernel start and end (moe_set_timing_events),
    with the median, p10 and p90 over the n calls."""
    import torch
    import bit_moe_amd as bm
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(n)]
    for s, e in evs:            # torch creates the HIP events on first record
        s.record()
        e.record()
    torch.cuda.synchronize()
    for i, (s, e) in enumerate(evs):
        bm.set_timing_events(s, e, which)
        step(i)
    bm.set_timing_events(None, None)
    torch.cuda.synchronize()
    d = sorted(s.elapsed_time(e) for s, e in evs)
    q = lambda f: d[min(len(d) - 1, int(f * (len(d) - 1) + 0.5))]
    return sum(d) / n, {"median_ms": q(0.5), "p10_ms": q(0.1), "p90_ms": q(0.9), "n": n}


def decode_b1(args, L, lays, fmt="2bit"):
    import torch
    import bit_moe_amd as bm
    import synth
    w = synth.WORKLOADS["decode_b1"].with_(fmt=fmt)
    R = 16
    xs_np, _ = synth.make_tokens(w.with_(T=R))
    xs = [torch.from_numpy(xs_np[i:i + 1].view("int16")).view(torch.bfloat16).cuda() for i in range(R)]
    ids = torch.empty((1, w.k), dtype=torch.int32, device="cuda")
    wt = torch.empty((1, w.k), dtype=torch.float32, device="cuda")
    y = torch.empty((1, w.H), dtype=torch.float32, device="cuda")
    ws = torch.empty(bm.workspace_bytes(lays[0], 1, bm.DECODE), dtype=torch.uint8, device="cuda")

    def step(i):
        lay, x = lays[i % len(lays)], xs[i % R]
        bm.forward_decode(lay, x, ids=ids, w=wt, y=y, ws=ws)

    ms, stats = time_steps(step, args.warmup, args.steps)
    n = min(args.steps, 100)
    gu_ms, gu_stats = time_kernel(step, n, bm.TIME_GATEUP)
    dn_ms, dn_stats = time_kernel(step, n, bm.TIME_DOWN)
    # the gate/up launch streams the routed gate/up blocks of the k experts
    # and, for 2-bit experts and k a power of two up to 16 (the shared
    # expert's rows split over the k workgroups of each panel), the shared
    # gate/up; the down launch the k experts' down blocks and the shared down
    eg, ed = expert_bytes(w)
    shared_in_gu = w.shared and fmt == "2bit" and w.k <= 16 and 64 % w.k == 0
    gu_bytes = w.k * eg + (2 * w.I * w.H * 2 if shared_in_gu else 0)
    dn_bytes = w.k * ed + w.I * w.H * 2
    step_bytes = w.k * (eg + ed) + 3 * w.I * w.H * 2 + w.E * w.H * 2
    return dict(ms=ms, stats=stats, gu_ms=gu_ms, gu_stats=gu_stats, gu_bytes=gu_bytes, dn_ms=dn_ms,
                dn_stats=dn_stats, dn_bytes=dn_bytes, step_bytes=step_bytes)


def decode_b16(args, lays):
    import torch
    import bit_moe_amd as bm
    import numpy as np
    import synth
    w = synth.WORKLOADS["decode_b16_zipf"]
    R = 4
    xs, lgs = [], []
    for r in range(R):
        wr = w.with_(seed=w.seed + 100 * r)
        x, _ = synth.make_tokens(wr)
        xs.append(torch.from_numpy(x.view("int16")).view(torch.bfloat16).cuda())
        lgs.append(torch.from_numpy(synth.zipf_logits(wr)).cuda())
    ids = torch.empty((w.T, w.k), dtype=torch.int32, device="cuda")
    wt = torch.empty((w.T, w.k), dtype=torch.float32, device="cuda")
    y = torch.empty((w.T, w.H), dtype=torch.float32, device="cuda")
    ws = torch.empty(bm.workspace_bytes(lays[0], w.T, bm.DECODE), dtype=torch.uint8, device="cuda")

    def step(i):
        lay, r = lays[i % len(lays)], i % R
        bm.topk(lgs[r], w.k, ids=ids, w=wt)
        bm.ffn_decode(lay, xs[r], ids, wt, y=y, ws=ws)

    ms, stats = time_steps(step, args.warmup, args.steps)
    # distinct experts per draw decide the bytes streamed
    d = np.mean([len(np.unique(bm.topk(l, w.k)[0].cpu().numpy())) for l in lgs])
    byts = d * w.I * (w.H // 256) * 66 * 2 + d * w.H * (w.I // 256) * 84 + 3 * w.I * w.H * 2
    return dict(ms=ms, stats=stats, distinct=float(d), bytes=float(byts))


def decode_small(args, lays, sizes=(2, 3, 4, 8)):
    """Tiny decode batches (speculative verification of 2-3 tokens, a few
    batched sessions): moe_forward_decode of T bf16 tokens with the routing
    computed on the GPU, the layer rotated as at batch 1."""
    import numpy as np
    import torch
    import bit_moe_amd as bm
    import synth
    w0 = synth.WORKLOADS["decode_b1"]
    eg, ed = expert_bytes(w0)
    out = {}
    for T in sizes:
        R = 4
        xs = []
        for r in range(R):
            x, _ = synth.make_tokens(w0.with_(T=T, seed=w0.seed + 1000 * T + r))
            xs.append(torch.from_numpy(x.view("int16")).view(torch.bfloat16).cuda())
        ids = torch.empty((T, w0.k), dtype=torch.int32, device="cuda")
        wt = torch.empty((T, w0.k), dtype=torch.float32, device="cuda")
        y = torch.empty((T, w0.H), dtype=torch.float32, device="cuda")
        ws = torch.empty(bm.workspace_bytes(lays[0], T, bm.DECODE), dtype=torch.uint8, device="cuda")

        def step(i):
            bm.forward_decode(lays[i % len(lays)], xs[i % R], ids=ids, w=wt, y=y, ws=ws)

        ms, stats = time_steps(step, args.warmup, args.steps)
        d = []
        for r in range(R):
            bm.forward_decode(lays[0], xs[r], ids=ids, w=wt, y=y, ws=ws)
            d.append(len(np.unique(ids.cpu().numpy())))
        d = float(np.mean(d))
        byts = d * (eg + ed) + 3 * w0.I * w0.H * 2 + w0.E * w0.H * 2
        out[f"T{T}"] = {"tokens": T, "us_per_step": ms * 1e3, "step_us": {k.replace("_ms", "_us"): v * 1e3 if
                                                                          k.endswith("_ms") else v
                                                                          for k, v in stats.items()},
                        "tokens_per_s": T / (ms * 1e-3), "distinct_experts": d, "hbm_bytes": byts,
                        "hbm_GBps": byts / (ms * 1e-3) / 1e9, "hbm_frac": byts / (ms * 1e-3) / HBM_PEAK}
        log(f"[bench] decode T={T} {ms * 1e3:.1f} us/step ({d:.1f} distinct experts, "
            f"{byts / (ms * 1e-3) / 1e9:.0f} GB/s)")
    return out


def issued_rows(counts, tile_rows=96):
    """Rows the prefill matrix-core kernels run per expert: each row tile of
    up to 96 rows runs in blocks of 32, so a tile of r rows issues
    32 ceil(r / 32)."""
    tot = 0
    for c in counts:
        c = int(c)
        full, tail = divmod(c, tile_rows)
        tot += full * tile_rows + (-(-tail // 32)) * 32
    return tot


def prefill_2k(args, lays, fmt="2bit"):
    import numpy as np
    import torch
    import bit_moe_amd as bm
    import synth
    w = synth.WORKLOADS["prefill_2k"].with_(fmt=fmt)
    x, _ = synth.make_tokens(w)
    xd = torch.from_numpy(x.view("int16")).view(torch.bfloat16).cuda()
    lay = routed_view(bm, w, lays[0])
    ids = torch.empty((w.T, w.k), dtype=torch.int32, device="cuda")
    wt = torch.empty((w.T, w.k), dtype=torch.float32, device="cuda")
    y = torch.empty((w.T, w.H), dtype=torch.float32, device="cuda")
    rws = torch.empty(bm.route_workspace_bytes(lay, w.T, bm.BF16), dtype=torch.uint8, device="cuda")
    ws = torch.empty(bm.workspace_bytes(lay, w.T, bm.PREFILL), dtype=torch.uint8, device="cuda")

    def step(i):
        bm.route(lay, xd, ids=ids, w=wt, ws=rws)
        bm.ffn_prefill(lay, xd, ids, wt, y=y, ws=ws)

    ms, stats = time_steps(step, args.prefill_warmup, args.prefill_steps)
    nk = max(5, min(20, args.prefill_steps))
    gu_ms, gu_stats = time_kernel(step, nk, bm.TIME_GATEUP)
    dn_ms, dn_stats = time_kernel(step, nk, bm.TIME_DOWN)
    counts = np.bincount(ids.cpu().numpy().ravel(), minlength=w.E)
    pairs = w.T * w.k
    rows_issued = issued_rows(counts)
    eg, ed = expert_bytes(w)
    active = int(np.count_nonzero(counts))
    return dict(ms=ms, stats=stats, flops=pairs * 3 * 2 * w.H * w.I, gu_bytes=active * eg, dn_bytes=active * ed,
                gu_ms=gu_ms, gu_stats=gu_stats, gu_flops=pairs * 2 * 2 * w.H * w.I,
                gu_flops_issued=rows_issued * 2 * 2 * w.H * w.I,
                dn_ms=dn_ms, dn_stats=dn_stats, dn_flops=pairs * 2 * w.H * w.I,
                dn_flops_issued=rows_issued * 2 * w.H * w.I)


def prefill_8k_zipf(args, lays):
    """8192 tokens with drawn Zipf(1.2) logits (the hottest experts get over a
    thousand rows, the coldest a few): top-k of the logits + the prefill FFN."""
    import numpy as np
    import torch
    import bit_moe_amd as bm
    import synth
    w = synth.WORKLOADS["prefill_8k_zipf"]
    x, _ = synth.make_tokens(w)
    xd = torch.from_numpy(x.view("int16")).view(torch.bfloat16).cuda()
    lg = torch.from_numpy(synth.zipf_logits(w)).cuda()
    lay = routed_view(bm, w, lays[0])
    ids = torch.empty((w.T, w.k), dtype=torch.int32, device="cuda")
    wt = torch.empty((w.T, w.k), dtype=torch.float32, device="cuda")
    y = torch.empty((w.T, w.H), dtype=torch.float32, device="cuda")
    ws = torch.empty(bm.workspace_bytes(lay, w.T, bm.PREFILL), dtype=torch.uint8, device="cuda")

    def step(i):
        bm.topk(lg, w.k, ids=ids, w=wt)
        bm.ffn_prefill(lay, xd, ids, wt, y=y, ws=ws)

    ms, stats = time_steps(step, args.prefill_warmup, args.prefill_steps)
    rows = np.bincount(ids.cpu().numpy().ravel(), minlength=w.E)
    flops = w.T * w.k * 3 * 2 * w.H * w.I
    return dict(ms=ms, stats=stats, flops=flops, rows_max=int(rows.max()), rows_min=int(rows.min()))


FP64_OPS_PEAK = 256 * 64 * 2.4e9   # unfused fp64 operations/s: 256 CUs x 64 lanes x 2.4 GHz

# fp64 operations of the IQ2X search per superblock, error terms only:
# 8 groups x 16 scales x 4 runs x 256 codebook rows x 8 weights x 4
# (db*g, difference, square, accumulate)
IQ2X_OPS_PER_SB = 8 * 16 * 4 * 256 * 8 * 4


def cache_bench(args, lays, slots=96, steps=48, warm=8):
    """Decode batch 16 with Zipf(1.1) routing drawn anew each step, routed
    experts served from a pool of `slots` HBM slots (of 256) over pinned host
    slabs: top-k on the GPU, ids to the host, the cache's map (copies of the
    missing experts on the stream), the decode FFN on the pool.  The step
    includes the device-to-host sync the host-side policy needs.  Returns
    tokens/s, hit rate, host-to-device bytes, and the bandwidth of a plain
    pinned copy of one expert's slabs (the roofline's peak)."""
    import numpy as np
    import torch
    import bit_moe_amd as bm
    import synth
    w = synth.WORKLOADS["decode_b16_zipf"]
    lay = lays[0]
    host = tuple(t.cpu().pin_memory() for t in lay.tensors[1:4])
    cache = bm.ExpertCache(lay, host, slots)
    R = steps + warm
    xs, lgs = [], []
    for r in range(R):
        wr = w.with_(seed=w.seed + 7000 + r)
        x, _ = synth.make_tokens(wr)
        xs.append(torch.from_numpy(x.view("int16")).view(torch.bfloat16).cuda())
        lgs.append(torch.from_numpy(synth.zipf_logits(wr)).cuda())
    ids = torch.empty((w.T, w.k), dtype=torch.int32, device="cuda")
    wt = torch.empty((w.T, w.k), dtype=torch.float32, device="cuda")
    y = torch.empty((w.T, w.H), dtype=torch.float32, device="cuda")
    ids_h = torch.empty((w.T, w.k), dtype=torch.int32).pin_memory()
    slot_d = torch.empty((w.T, w.k), dtype=torch.int32, device="cuda")
    ws = torch.empty(bm.workspace_bytes(cache.layer, w.T, bm.DECODE), dtype=torch.uint8, device="cuda")
    copied = [0]

    def step(i):
        bm.topk(lgs[i], w.k, ids=ids, w=wt)
        ids_h.copy_(ids)                               # synchronous: the policy runs on the host
        sl, n = cache.map(ids_h)
        copied[0] += n
        slot_d.copy_(sl, non_blocking=True)
        bm.ffn_decode(cache.layer, xs[i], slot_d, wt, y=y, ws=ws)

    for i in range(warm):
        step(i)
    torch.cuda.synchronize()
    h0, m0, _ = cache.stats()
    copied[0] = 0
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    t0.record()
    for i in range(warm, R):
        step(i)
    t1.record()
    torch.cuda.synchronize()
    ms = t0.elapsed_time(t1) / steps
    h1, m1, _ = cache.stats()
    cache.close()
    eb = 2 * w.I * (w.H // 256) * 66 + w.H * (w.I // 256) * 84          # one expert's slabs
    # a plain pinned host-to-device copy of the same size as one expert's slabs
    src = torch.empty(eb, dtype=torch.uint8).pin_memory()
    dst = torch.empty(eb, dtype=torch.uint8, device="cuda")
    c0, c1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    dst.copy_(src, non_blocking=True)
    torch.cuda.synchronize()
    c0.record()
    for _ in range(20):
        dst.copy_(src, non_blocking=True)
    c1.record()
    torch.cuda.synchronize()
    copy_bw = 20 * eb / (c0.elapsed_time(c1) * 1e-3)
    hits, misses = h1 - h0, m1 - m0
    return dict(ms=ms, slots=slots, steps=steps, hits=hits, misses=misses, copied=copied[0], expert_bytes=eb,
                h2d_bytes_per_step=copied[0] * eb / steps, copy_bw=copy_bw)


def quantize_bench(args):
    """The quantizer on one full expert tensor per format (2048 x 7168 gate/up
    weights to IQ2X, 7168 x 2048 down weights to Q2K: 57344 superblocks
    each), synthetic N(0, 1/(10.6 sqrt(K))) weights resident in HBM."""
    import numpy as np
    import torch
    import bit_moe_amd as bm
    import synth
    n = 2048 * 7168 // 256
    rng = np.random.default_rng(7)
    w = torch.from_numpy((rng.standard_normal(n * 256) / (10.6 * np.sqrt(7168))).astype(np.float32)).cuda()
    grid = torch.from_numpy(synth.make_layer(synth.WORKLOADS["decode_b1"]).grid()).cuda()
    oi = torch.empty((n, 66), dtype=torch.uint8, device="cuda")
    oq = torch.empty((n, 84), dtype=torch.uint8, device="cuda")
    om = torch.empty((n * 8, 17), dtype=torch.uint8, device="cuda")
    ms_i, st_i = time_steps(lambda i: bm.quantize_iq2x(w, grid, out=oi), 1, 5)
    ms_q, st_q = time_steps(lambda i: bm.quantize_q2k(w, out=oq), 2, 20)
    ms_m, st_m = time_steps(lambda i: bm.quantize_mxfp4(w, out=om), 2, 20)
    return dict(n=n, ms_iq2x=ms_i, ms_q2k=ms_q, ms_mxfp4=ms_m, st_iq2x=st_i, st_q2k=st_q, st_mxfp4=st_m,
                w=w.cpu().numpy(), grid=grid.cpu().numpy())


def quantize_cpu_baseline(w, grid, target_s):
    """The oracle's encoder (all host threads) on a bounded sample of the
    same tensor's superblocks, IQ2X then Q2K."""
    import numpy as np
    import oracle
    out = {}
    for fmt, first in (("iq2x", 64), ("q2k", 4096), ("mxfp4", 4096)):
        nb, spent = first, 0.0
        while True:
            x = np.ascontiguousarray(w[:nb * 256])
            t0 = time.perf_counter()
            if fmt == "iq2x":
                oracle.quantize_iq2x(x, grid)
            elif fmt == "q2k":
                oracle.quantize_q2k(x)
            else:
                oracle.quantize_mxfp4(x)
            spent = time.perf_counter() - t0
            if spent >= target_s / 4 or nb * 256 * 2 > w.size:
                break
            nb *= 2
        out[fmt] = dict(value=nb * 256 / spent, unit="weights/s", cores=oracle.max_threads(), cpu=cpu_model(),
                        kind="oracle", sample=f"the first {nb} superblocks of the tensor, {spent:.2f} s")
    return out


def cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(name, target_s, max_tokens=400):
    """The oracle as it stands (plain fp64 C, all host threads) on a bounded
    sample of one workload's tokens, one token at a time until about target_s
    seconds of oracle time: routing (computed or drawn logits) and the layer
    per token.  Expert slabs are generated (untimed) before the token that
    first uses them."""
    import numpy as np
    import oracle
    import synth
    w = synth.WORKLOADS[name]
    L = synth.make_layer(w)
    T = min(max_tokens, w.T) if w.routing == "zipf" else max_tokens
    x, _ = synth.make_tokens(w.with_(T=T))
    zl = synth.zipf_logits(w, T=T).astype(np.float64) if w.routing == "zipf" else None
    grid, router, shared = L.grid(), L.router(), L.shared()
    gate, up, down = {}, {}, {}
    spent, n = 0.0, 0
    while n < T and (spent < target_s or n < 4):
        xt = x[n:n + 1]
        t0 = time.perf_counter()
        ids, wt = oracle.topk(zl[n:n + 1], w.k) if zl is not None else oracle.route(xt, router, w.k)
        spent += time.perf_counter() - t0
        for e in (int(v) for v in np.unique(ids)):
            if e not in gate:
                gate[e], up[e], down[e] = L.gate(e), L.up(e), L.down(e)
        t0 = time.perf_counter()
        oracle.moe_ffn(w.H, w.I, w.E, w.k, grid, gate, up, down, shared, xt, ids, wt)
        spent += time.perf_counter() - t0
        n += 1
    what = {"decode_b1": "the batch-1 decode workload (routing + 8 routed experts + shared expert each)",
            "decode_b16_zipf": "the 16-token Zipf(1.1) decode batch (top-k of the drawn logits + 8 routed "
                               "experts + shared expert each)",
            "prefill_2k": "the 2048-token prefill chunk (routing + 8 routed experts each)"}[name]
    return dict(value=n / spent, unit="tokens/s", cores=oracle.max_threads(), cpu=cpu_model(), kind="oracle",
                sample=f"{n} tokens of {what}, fp64, {spent:.1f} s of oracle time")


def copy_calibration(nbytes=1 << 30, reps=5):
    """A plain device copy of known size, for scaling the FETCH_SIZE and
    WRITE_SIZE counters (run under rocprofv3 --pmc)."""
    import torch
    a = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    b = torch.empty_like(a)
    a.fill_(1)
    for _ in range(reps):
        b.copy_(a)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes": nbytes, "reps": reps}), flush=True)


def _pmc_per_kernel(dirname, counter):
    """{kernel name: average counter value per dispatch} from a rocprofv3
    --pmc output directory (sqlite database)."""
    import glob
    import sqlite3
    out = {}
    for db in glob.glob(os.path.join(dirname, "**", "*.db"), recursive=True):
        c = sqlite3.connect(db)
        q = ("select kernel_name, value from counters_collection where counter_name = ?")
        acc = {}
        for name, v in c.execute(q, (counter,)):
            acc.setdefault(name, []).append(v)
        for name, vs in acc.items():
            out[name] = sum(vs) / len(vs)
    return out


def source_digest():
    import hashlib
    h = hashlib.sha256()
    for f in ("decode.hip", "common.h", "device_util.h", "plan.cpp", "host.h"):
        with open(os.path.join(ROOT, "bit_moe_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def summarize_traffic(fetch_dir, write_dir, cfetch_dir, cwrite_dir, copy_bytes):
    """Text summary: HBM bytes per dispatch of each decode kernel, the
    counters scaled by what they read for the plain copy."""
    fetch, write = _pmc_per_kernel(fetch_dir, "FETCH_SIZE"), _pmc_per_kernel(write_dir, "WRITE_SIZE")
    cf = max(v for k, v in _pmc_per_kernel(cfetch_dir, "FETCH_SIZE").items() if "copyBuffer" in k)
    cw = max(v for k, v in _pmc_per_kernel(cwrite_dir, "WRITE_SIZE").items() if "copyBuffer" in k)
    f_scale, w_scale = copy_bytes / (cf * 1024.0), copy_bytes / (cw * 1024.0)
    lines = [f"source_digest {source_digest()}",
             f"copy_calibration bytes {copy_bytes} FETCH_SIZE_KiB {cf:.1f} WRITE_SIZE_KiB {cw:.1f} "
             f"fetch_scale {f_scale:.4f} write_scale {w_scale:.4f}"]
    for k in sorted(fetch):
        if "k_dec" not in k:
            continue
        fb, wb = fetch[k] * 1024.0 * f_scale, write.get(k, 0.0) * 1024.0 * w_scale
        name = k[k.index("k_dec"):].split("(")[0].replace(" ", "")
        lines.append(f"kernel {name} fetch_bytes {fb:.0f} write_bytes {wb:.0f} "
                     f"traffic_bytes {fb + wb:.0f}")
    return "\n".join(lines)


def summarize_kernels(trace_dir):
    """Per-kernel launch count and average / min / max duration (us) from a
    rocprofv3 --kernel-trace output directory of a default bench run, grouped
    by bench phase, name and grid.  Phases follow the run's order: layer set-up
    (packing) until the first decode launch, decode_b1 until the batch-16 step's
    first top-k, decode_b16 (the decode batch also runs prefill kernels, for
    its multi-token experts) until the first decode launch not preceded by a
    top-k, decode_small (2 to 8 tokens) until the prefill step's router GEMM, prefill_2k
    until the 8192-token step's top-k, prefill_8k until the expert cache's
    first decode launch, expert_cache until the quantizer, quantize until the
    MXFP4 layer's packing, then mxfp4_decode_b1 from its first decode launch
    and mxfp4_prefill_2k from its router GEMM."""
    import glob
    import sqlite3
    rows = {}
    for db in glob.glob(os.path.join(trace_dir, "**", "*.db"), recursive=True):
        c = sqlite3.connect(db)
        phase, prev = "setup", ""
        for name, gx, t0, t1 in c.execute("select name, grid_x, start, end from kernels order by start"):
            if phase == "setup" and "k_dec_front" in name:
                phase = "decode_b1"
            elif phase == "decode_b1" and ("k_topk" in name or "k_dec_mid" in name):
                phase = "decode_b16"
            elif phase == "decode_b16" and "k_dec_front" in name and "k_topk" not in prev:
                phase = "decode_small"
            elif phase in ("decode_b16", "decode_small") and "k_router_splitk" in name:
                phase = "prefill_2k"
            elif phase == "prefill_2k" and "k_topk" in name and "k_topk_sum" not in name:
                phase = "prefill_8k"
            elif phase == "prefill_8k" and "k_dec_front" in name:
                phase = "expert_cache"
            elif phase == "expert_cache" and "k_quant" in name:
                phase = "quantize"
            elif phase == "quantize" and "k_pack_mxfp4" in name:
                phase = "mxfp4_setup"
            elif phase == "mxfp4_setup" and "k_dec_front" in name:
                phase = "mxfp4_decode_b1"
            elif phase == "mxfp4_decode_b1" and "k_router_splitk" in name:
                phase = "mxfp4_prefill_2k"
            prev = name
            r = rows.setdefault((phase, name, gx), [0, 0.0, float("inf"), 0.0])
            d = (t1 - t0) / 1e3
            r[0] += 1
            r[1] += d
            r[2] = min(r[2], d)
            r[3] = max(r[3], d)
    out = [f"{'phase':<16} {'calls':>6} {'avg_us':>10} {'min_us':>10} {'max_us':>10} {'grid':>10}  kernel"]
    order = {p: i for i, p in enumerate(("setup", "decode_b1", "decode_b16", "decode_small", "prefill_2k", "prefill_8k",
                                         "expert_cache", "quantize", "mxfp4_setup", "mxfp4_decode_b1",
                                         "mxfp4_prefill_2k"))}
    for (phase, name, gx), (n, tot, mn, mx) in sorted(rows.items(), key=lambda kv: (order[kv[0][0]], -kv[1][1])):
        short = name[name.index("k_"):].split("(")[0] if "k_" in name else name.split("(")[0]
        out.append(f"{phase:<16} {n:6d} {tot / n:10.2f} {mn:10.2f} {mx:10.2f} {gx:10d}  {short}")
    return "\n".join(out)


def summarize_mfma(pmc_dir):
    """Per-kernel fp16/bf16 MFMA work from SQ_INSTS_VALU_MFMA_MOPS_F16/_BF16
    (multiply-accumulates in units of 512, i.e. 1024 flops) over the kernel's
    duration in the same run; the work includes any padding of partial tiles."""
    import glob
    import sqlite3
    db = glob.glob(os.path.join(pmc_dir, "*.db"))[0]
    c = sqlite3.connect(db)
    mops = {}
    for kn, cn, v in c.execute("select kernel_name, counter_name, sum(value) from counters_collection "
                               "group by dispatch_id, counter_name"):
        if "MFMA_MOPS" in cn:
            mops.setdefault(kn, []).append(v)
    dur = {}
    for kn, d in c.execute("select name, end - start from kernels"):
        dur.setdefault(kn, []).append(d)
    lines = [f"{'kernel':40s} {'calls':>5s} {'avg_us':>9s} {'mfma_TFLOP':>11s} {'TFLOP/s':>9s} {'frac_2.5PF':>10s}"]
    for kn, v in sorted(mops.items()):
        if not any(x > 0 for x in v) or kn not in dur:
            continue
        fl = sum(v) / len(v) * 1024.0
        us = sum(dur[kn]) / len(dur[kn]) / 1e3
        name = kn.replace("(anonymous namespace)::", "").split("(")[0][:40]
        lines.append(f"{name:40s} {len(v):5d} {us:9.1f} {fl / 1e12:11.3f} {fl / (us * 1e-6) / 1e12:9.1f} "
                     f"{fl / (us * 1e-6) / BF16_PEAK:10.3f}")
    return "\n".join(lines)


def summarize_counters(dirs, only=("k_pf_", "k_mx_", "k_dec_", "k_combine", "k_shared")):
    """Per-kernel average per dispatch of every counter collected in one or
    more rocprofv3 --pmc output directories (one pass each), one row per
    kernel with the counters as columns, plus the kernels' average
    durations from the same runs."""
    import glob
    import sqlite3
    vals, durs = {}, {}
    for d in dirs:
        for db in glob.glob(os.path.join(d, "**", "*.db"), recursive=True):
            c = sqlite3.connect(db)
            per = {}
            for kn, disp, cn, v in c.execute("select kernel_name, dispatch_id, counter_name, sum(value) "
                                             "from counters_collection group by dispatch_id, counter_name"):
                per.setdefault((kn, cn), []).append(v)
            for (kn, cn), v in per.items():
                vals.setdefault(kn, {})[cn] = sum(v) / len(v)
            try:
                for kn, t in c.execute("select name, end - start from kernels"):
                    durs.setdefault(kn, []).append(t)
            except sqlite3.Error:
                pass
    out = []
    for kn in sorted(vals):
        short = kn.replace("(anonymous namespace)::", "").split("(")[0]
        if only and not any(o in short for o in only):
            continue
        us = sum(durs.get(kn, [0])) / max(1, len(durs.get(kn, []))) / 1e3
        out.append(f"kernel {short} avg_us {us:.1f}")
        for cn in sorted(vals[kn]):
            out.append(f"  {cn} {vals[kn][cn]:.6g}")
    return "\n".join(out)


def traffic_from_profile(kernel):
    """HBM bytes per launch of `kernel` from the committed counter summary,
    or None when the decode sources have changed since it was taken."""
    p = os.path.join(ROOT, "profiles", "traffic_k_dec_decode_b1.txt")
    if not os.path.exists(p):
        return None
    lines = open(p).read().splitlines()
    dig = [l.split()[1] for l in lines if l.startswith("source_digest")]
    if not dig or dig[0] != source_digest():
        return None
    for l in lines:
        f = l.split()
        if f and f[0] == "kernel" and f[1] == kernel:
            return float(f[f.index("traffic_bytes") + 1])
    return None


def mxfp4_bench(args):
    """The MXFP4 routed-expert variant at the decode batch-1 and 2048-token
    prefill shapes (same router, shared expert and routing as the 2-bit
    lines)."""
    import torch
    import synth
    w = synth.WORKLOADS["decode_b1"].with_(fmt="mxfp4")
    L, lays = build_layer(w, args.copies)
    r = decode_b1(args, L, lays, fmt="mxfp4")
    usd = lambda st: {k.replace("_ms", "_us"): (v * 1e3 if k.endswith("_ms") else v) for k, v in st.items()}
    gu_bw = r["gu_bytes"] / (r["gu_ms"] * 1e-3)
    dn_bw = r["dn_bytes"] / (r["dn_ms"] * 1e-3)
    log(f"[bench] mxfp4 decode_b1 {r['ms'] * 1e3:.1f} us/step, gate/up {r['gu_ms'] * 1e3:.1f} us "
        f"({gu_bw / 1e9:.0f} GB/s), down {r['dn_ms'] * 1e3:.1f} us")
    res = {"workload": "MXFP4 routed experts (OCP Microscaling: E2M1 elements, E8M0 scale per 32 weights) at "
                       "H7168, I2048, 256 experts top-8; decode: moe_forward_decode of one bf16 token with the bf16 "
                       "shared expert; prefill: route + moe_ffn_prefill of 2048 bf16 tokens",
           "decode_b1": {"tokens_per_s": 1.0 / (r["ms"] * 1e-3), "us_per_step": r["ms"] * 1e3,
                         "step_us": usd(r["stats"]), "step_hbm_bytes": r["step_bytes"],
                         "step_hbm_GBps": r["step_bytes"] / (r["ms"] * 1e-3) / 1e9,
                         "roofline": {"bound": "hbm", "kernel": "k_dec_gateup (MXFP4)", "unit": "GB/s",
                                      "achieved": gu_bw / 1e9, "peak": HBM_PEAK / 1e9, "frac": gu_bw / HBM_PEAK,
                                      "kernel_us": r["gu_ms"] * 1e3, "algorithmic_bytes": r["gu_bytes"],
                                      "traffic": None,
                                      "down_kernel": {"kernel": "k_dec_down (MXFP4)", "achieved": dn_bw / 1e9,
                                                      "frac": dn_bw / HBM_PEAK, "kernel_us": r["dn_ms"] * 1e3,
                                                      "algorithmic_bytes": r["dn_bytes"]}}}}
    del lays[1:]
    torch.cuda.empty_cache()
    pf = prefill_2k(args, lays, fmt="mxfp4")
    tfs = lambda f, ms: f / (ms * 1e-3) / 1e12
    res["prefill_2k"] = {
        "tokens_per_s": 2048 / (pf["ms"] * 1e-3), "ms_per_step": pf["ms"], "step_ms": pf["stats"],
        "routed_TFLOPs": tfs(pf["flops"], pf["ms"]), "mfma_frac": pf["flops"] / (pf["ms"] * 1e-3) / BF16_PEAK,
        "roofline": [
            {"bound": "mfma", "kernel": kname, "unit": "TFLOP/s", "peak": BF16_PEAK / 1e12,
             "achieved": tfs(pf[f + "_flops"], pf[f + "_ms"]),
             "frac": tfs(pf[f + "_flops"], pf[f + "_ms"]) * 1e12 / BF16_PEAK,
             "issued_frac": tfs(pf[f + "_flops_issued"], pf[f + "_ms"]) * 1e12 / BF16_PEAK,
             "kernel_us": pf[f + "_ms"] * 1e3, "algorithmic_flops": pf[f + "_flops"], "traffic": None,
             # at about 64 rows per expert the MXFP4 weights (17/32 B per weight) make this kernel's
             # intensity 2 x 64 / (17/32) = 241 FLOP/B, below the 312 FLOP/B ridge: HBM binds first
             "weight_bytes": pf[f + "_bytes"], "hbm_GBps": pf[f + "_bytes"] / (pf[f + "_ms"] * 1e-3) / 1e9,
             "hbm_frac": pf[f + "_bytes"] / (pf[f + "_ms"] * 1e-3) / HBM_PEAK}
            for kname, f in (("k_mx_gateup", "gu"), ("k_mx_down", "dn"))]}
    log(f"[bench] mxfp4 prefill_2k {pf['ms']:.2f} ms/step, gate/up {pf['gu_ms'] * 1e3:.0f} us, "
        f"down {pf['dn_ms'] * 1e3:.0f} us")
    del lays
    torch.cuda.empty_cache()
    return res


def main():
    args = parse()
    if args.summarize_kernels:
        print(summarize_kernels(args.summarize_kernels))
        return
    if args.summarize_traffic:
        print(summarize_traffic(*args.summarize_traffic, copy_bytes=1 << 30))
        return
    if args.summarize_mfma:
        print(summarize_mfma(args.summarize_mfma))
        return
    if args.summarize_counters:
        print(summarize_counters(args.summarize_counters))
        return
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (got --gpus {args.gpus}); this build has no "
              f"multi-GPU path. Run with --gpus 1.", file=sys.stderr)
        sys.exit(2)
    import torch
    import bit_moe_amd as bm
    import synth
    bm.lib()
    assert torch.cuda.is_available(), "bench.py needs a GPU"
    if args.copy_calibration:
        copy_calibration()
        return
    if args.prefill_only:
        _, lays = build_layer(synth.WORKLOADS["decode_b1"].with_(fmt=args.fmt), 1)
        pf = prefill_2k(args, lays, fmt=args.fmt)
        log(f"[bench] {args.fmt} prefill_2k {pf['ms']:.2f} ms/step, gate/up {pf['gu_ms'] * 1e3:.1f} us, "
            f"down {pf['dn_ms'] * 1e3:.1f} us")
        return
    w = synth.WORKLOADS["decode_b1"]
    L, lays = build_layer(w, args.copies)
    r = decode_b1(args, L, lays)
    log(f"[bench] decode_b1 {r['ms'] * 1e3:.1f} us/step (median {r['stats']['median_ms'] * 1e3:.1f}), "
        f"gate/up {r['gu_ms'] * 1e3:.1f} us, down {r['dn_ms'] * 1e3:.1f} us")
    gu_bw = r["gu_bytes"] / (r["gu_ms"] * 1e-3)
    dn_bw = r["dn_bytes"] / (r["dn_ms"] * 1e-3)
    us = lambda st: {k: (v * 1e3 if k.endswith("_ms") else v) for k, v in st.items()}
    usd = lambda st: {k.replace("_ms", "_us"): v for k, v in us(st).items()}
    out = {
        "metric": "MoE-layer tokens/s: decode HBM GB/s (%peak) + prefill MFMA TFLOP/s (%peak)",
        "value": 1.0 / (r["ms"] * 1e-3),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": r["ms"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "decode batch 1: 1 token, H7168, I2048, 256 routed experts top-8, "
                               "IQ2X up/gate + Q2K down, bf16 router and shared expert",
                   "tokens_per_step": 1, "layer_copies_rotated": args.copies,
                   "step_hbm_bytes": r["step_bytes"],
                   "step_hbm_GBps": r["step_bytes"] / (r["ms"] * 1e-3) / 1e9,
                   "step_us": usd(r["stats"])},
        "roofline": {"bound": "hbm", "kernel": "k_dec_gateup",
                     "achieved": gu_bw / 1e9, "peak": HBM_PEAK / 1e9, "unit": "GB/s",
                     "frac": gu_bw / HBM_PEAK, "traffic": traffic_from_profile("k_dec_gateup<0,1,0>"),
                     "kernel_us": r["gu_ms"] * 1e3, "kernel_us_dist": usd(r["gu_stats"]),
                     "algorithmic_bytes": r["gu_bytes"],
                     "down_kernel": {"kernel": "k_dec_down", "achieved": dn_bw / 1e9, "frac": dn_bw / HBM_PEAK,
                                     "kernel_us": r["dn_ms"] * 1e3, "algorithmic_bytes": r["dn_bytes"],
                                     "traffic": traffic_from_profile("k_dec_down<0,0>")}},
    }
    if not args.no_extra:
        b16 = decode_b16(args, lays)
        out["decode_b16_zipf"] = {"tokens_per_s": 16 / (b16["ms"] * 1e-3), "ms_per_step": b16["ms"],
                                  "step_us": usd(b16["stats"]),
                                  "distinct_experts": b16["distinct"],
                                  "hbm_GBps": b16["bytes"] / (b16["ms"] * 1e-3) / 1e9,
                                  "hbm_frac": b16["bytes"] / (b16["ms"] * 1e-3) / HBM_PEAK,
                                  "note": "step = top-k of drawn Zipf(1.1) logits + decode FFN"}
        log(f"[bench] decode_b16 {b16['ms'] * 1e3:.1f} us/step")
        out["decode_small"] = dict(decode_small(args, lays),
                                   note="moe_forward_decode of T bf16 tokens, routing on the GPU; HBM bytes over the "
                                        "realised distinct experts + shared expert + router")
        del lays[1:]
        torch.cuda.empty_cache()
        pf = prefill_2k(args, lays)
        tfs = lambda f, ms: f / (ms * 1e-3) / 1e12
        out["prefill_2k"] = {
            "tokens_per_s": 2048 / (pf["ms"] * 1e-3), "ms_per_step": pf["ms"], "step_ms": pf["stats"],
            "routed_TFLOPs": tfs(pf["flops"], pf["ms"]),
            "mfma_frac": pf["flops"] / (pf["ms"] * 1e-3) / BF16_PEAK,
            "roofline": [
                {"bound": "mfma", "kernel": "k_pf_gateup", "unit": "TFLOP/s", "peak": BF16_PEAK / 1e12,
                 "achieved": tfs(pf["gu_flops"], pf["gu_ms"]), "frac": tfs(pf["gu_flops"], pf["gu_ms"]) * 1e12 / BF16_PEAK,
                 "issued_frac": tfs(pf["gu_flops_issued"], pf["gu_ms"]) * 1e12 / BF16_PEAK,
                 "kernel_us": pf["gu_ms"] * 1e3, "kernel_us_dist": usd(pf["gu_stats"]),
                 "algorithmic_flops": pf["gu_flops"], "issued_flops": pf["gu_flops_issued"], "traffic": None},
                {"bound": "mfma", "kernel": "k_pf_down", "unit": "TFLOP/s", "peak": BF16_PEAK / 1e12,
                 "achieved": tfs(pf["dn_flops"], pf["dn_ms"]), "frac": tfs(pf["dn_flops"], pf["dn_ms"]) * 1e12 / BF16_PEAK,
                 "issued_frac": tfs(pf["dn_flops_issued"], pf["dn_ms"]) * 1e12 / BF16_PEAK,
                 "kernel_us": pf["dn_ms"] * 1e3, "kernel_us_dist": usd(pf["dn_stats"]),
                 "algorithmic_flops": pf["dn_flops"], "issued_flops": pf["dn_flops_issued"], "traffic": None}]}
        log(f"[bench] prefill_2k {pf['ms']:.2f} ms/step, gate/up {pf['gu_ms'] * 1e3:.0f} us, "
            f"down {pf['dn_ms'] * 1e3:.0f} us")
        p8 = prefill_8k_zipf(args, lays)
        out["prefill_8k_zipf"] = {"tokens_per_s": 8192 / (p8["ms"] * 1e-3), "ms_per_step": p8["ms"],
                                  "step_ms": p8["stats"],
                                  "routed_TFLOPs": p8["flops"] / (p8["ms"] * 1e-3) / 1e12,
                                  "mfma_frac": p8["flops"] / (p8["ms"] * 1e-3) / BF16_PEAK,
                                  "rows_per_expert_max": p8["rows_max"], "rows_per_expert_min": p8["rows_min"],
                                  "note": "step = top-k of drawn Zipf(1.2) logits + prefill FFN"}
        log(f"[bench] prefill_8k_zipf {p8['ms']:.2f} ms/step")
        cb = cache_bench(args, lays)
        h2d = cb["h2d_bytes_per_step"] / (cb["ms"] * 1e-3)
        out["expert_cache"] = {
            "workload": f"decode batch 16, Zipf(1.1) routing drawn per step, {cb['slots']} HBM slots of 256 experts "
                        "over pinned host slabs; step = top-k, ids to host, cache map (copies of misses), decode FFN",
            "tokens_per_s": 16 / (cb["ms"] * 1e-3), "ms_per_step": cb["ms"], "steps": cb["steps"],
            "hit_rate": cb["hits"] / max(1, cb["hits"] + cb["misses"]), "experts_copied_per_step": cb["copied"] / cb["steps"],
            "roofline": {"bound": "pcie", "unit": "GB/s", "achieved": h2d / 1e9, "peak": cb["copy_bw"] / 1e9,
                         "frac": h2d / cb["copy_bw"], "peak_note": "a plain pinned host-to-device copy of one "
                         "expert's slabs, measured in the same run", "traffic": None}}
        log(f"[bench] expert_cache {cb['ms']:.3f} ms/step, hit rate {out['expert_cache']['hit_rate']:.3f}, "
            f"{cb['copied'] / cb['steps']:.1f} experts copied per step, H2D {h2d / 1e9:.1f} GB/s "
            f"(plain copy {cb['copy_bw'] / 1e9:.1f} GB/s)")
        qb = quantize_bench(args)
        iq_ops = qb["n"] * IQ2X_OPS_PER_SB / (qb["ms_iq2x"] * 1e-3)
        q_bytes = qb["n"] * (256 * 4 + 84) / (qb["ms_q2k"] * 1e-3)
        m_bytes = qb["n"] * 8 * (32 * 4 + 17) / (qb["ms_mxfp4"] * 1e-3)
        out["quantize"] = {
            "workload": "one 2048 x 7168 expert tensor of fp32 weights (57344 superblocks) per format",
            "iq2x": {"weights_per_s": qb["n"] * 256 / (qb["ms_iq2x"] * 1e-3), "ms": qb["ms_iq2x"],
                     "ms_dist": qb["st_iq2x"],
                     "roofline": {"bound": "alu", "unit": "Gop/s (fp64, unfused)", "achieved": iq_ops / 1e9,
                                  "peak": FP64_OPS_PEAK / 1e9, "frac": iq_ops / FP64_OPS_PEAK,
                                  "ops_per_superblock": IQ2X_OPS_PER_SB, "traffic": None}},
            "q2k": {"weights_per_s": qb["n"] * 256 / (qb["ms_q2k"] * 1e-3), "ms": qb["ms_q2k"],
                    "ms_dist": qb["st_q2k"],
                    "roofline": {"bound": "hbm", "unit": "GB/s", "achieved": q_bytes / 1e9, "peak": HBM_PEAK / 1e9,
                                 "frac": q_bytes / HBM_PEAK, "bytes_per_superblock": 256 * 4 + 84,
                                 "traffic": None}},
            "mxfp4": {"weights_per_s": qb["n"] * 256 / (qb["ms_mxfp4"] * 1e-3), "ms": qb["ms_mxfp4"],
                      "ms_dist": qb["st_mxfp4"],
                      "roofline": {"bound": "hbm", "unit": "GB/s", "achieved": m_bytes / 1e9,
                                   "peak": HBM_PEAK / 1e9, "frac": m_bytes / HBM_PEAK,
                                   "bytes_per_block": 32 * 4 + 17, "traffic": None}}}
        log(f"[bench] quantize iq2x {qb['ms_iq2x']:.2f} ms, q2k {qb['ms_q2k']:.3f} ms, "
            f"mxfp4 {qb['ms_mxfp4']:.3f} ms per tensor")
    if not args.no_extra:
        del lays, L
        torch.cuda.empty_cache()
        out["mxfp4"] = mxfp4_bench(args)
    if not args.no_cpu_baseline:
        if not args.no_extra:
            for fmt, cb in quantize_cpu_baseline(qb["w"], qb["grid"], args.cpu_seconds / 2).items():
                out["quantize"][fmt]["cpu_baseline"] = cb
                log(f"[bench] cpu baseline quantize {fmt} {cb['value']:.3g} weights/s")
        out["cpu_baseline"] = cpu_baseline("decode_b1", args.cpu_seconds)
        log(f"[bench] cpu baseline {out['cpu_baseline']['value']:.3f} tokens/s")
        if not args.no_extra:
            for name in ("decode_b16_zipf", "prefill_2k"):
                out[name]["cpu_baseline"] = cb = cpu_baseline(name, args.cpu_seconds / 2)
                log(f"[bench] cpu baseline {name} {cb['value']:.3f} tokens/s")
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
