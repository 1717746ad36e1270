#!/usr/bin/env python3
"""Throughput of the 2-bit routed-expert MoE layer on one MI355X.

One step = one pass of the whole hot path over one batch held in HBM:
router logits + top-k/renormalise (moe_route), then moe_ffn_decode
(bucketing, fused IQ2X gate/up dequant-GEMV + SwiGLU, fused Q2K down
dequant-GEMV, gate-weighted combine, bf16 shared expert).

Workload of the headline line: one decode token at DeepSeek-V4-Flash MoE
shapes (H 7168, I 2048, 256 routed experts, top-8, one bf16 shared expert),
seeded synthetic weights.  To keep timed calls out of the 256 MB MALL, the
steps rotate over --copies independent device copies of the layer and over
16 different token rows.  Extra objects report the 16-token Zipf decode
batch and the 2048-token prefill chunk (grouped bf16-MFMA GEMMs).

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
BF16_PEAK = 2.5e15         # FLOP/s, dense bf16 MFMA


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--copies", type=int, default=8, help="layer copies rotated to defeat MALL")
    ap.add_argument("--prefill-steps", type=int, default=10)
    ap.add_argument("--cpu-tokens", type=int, default=8, help="oracle sample size (tokens)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-extra", action="store_true", help="skip the b16 and prefill lines")
    return ap.parse_args()


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def build_layer(w, copies):
    import torch
    import bit_moe_amd as bm
    import synth
    L = synth.make_layer(w)
    t0 = time.time()
    lay = bm.layer_from_canonical(w.H, w.I, w.E, w.k, L.router(), L.gate_all(), L.up_all(),
                                  L.down_all(), L.grid(), L.shared())
    torch.cuda.synchronize()
    log(f"[bench] layer generated+packed in {time.time() - t0:.1f}s")
    lays = [lay]
    for _ in range(copies - 1):
        t = [x.clone() for x in lay.tensors]
        sh = tuple(t[5:8]) if lay.has_shared else None
        lays.append(bm.Layer(w.H, w.I, w.E, w.k, t[0], t[1], t[2], t[3], t[4], sh))
    torch.cuda.synchronize()
    return L, lays


def time_steps(step, warmup, steps):
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
    return a.elapsed_time(b) / steps      # ms per step


def time_dominant(step, n):
    """Average duration of the gate/up kernel, from HIP events the library
    records around that launch on its stream."""
    import torch
    import bit_moe_amd as bm
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(n)]
    for s, e in evs:            # torch creates the HIP events on first record
        s.record()
        e.record()
    torch.cuda.synchronize()
    for i, (s, e) in enumerate(evs):
        bm.set_timing_events(s, e)
        step(i)
    bm.set_timing_events(None, None)
    torch.cuda.synchronize()
    return sum(s.elapsed_time(e) for s, e in evs) / n


def decode_b1(args, L, lays):
    import torch
    import bit_moe_amd as bm
    import synth
    w = synth.WORKLOADS["decode_b1"]
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

    ms = time_steps(step, args.warmup, args.steps)
    gu_ms = time_dominant(step, min(args.steps, 100))
    # the timed launch streams the routed gate/up blocks of the k experts
    gu_bytes = w.k * (2 * w.I * (w.H // 256) * 66)
    step_bytes = w.k * (2 * w.I * (w.H // 256) * 66 + w.H * (w.I // 256) * 84) + 3 * w.I * w.H * 2 + w.E * w.H * 2
    return dict(ms=ms, gu_ms=gu_ms, gu_bytes=gu_bytes, step_bytes=step_bytes)


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

    ms = time_steps(step, args.warmup, args.steps)
    # distinct experts per draw decide the bytes streamed
    d = np.mean([len(np.unique(bm.topk(l, w.k)[0].cpu().numpy())) for l in lgs])
    byts = d * w.I * (w.H // 256) * 66 * 2 + d * w.H * (w.I // 256) * 84 + 3 * w.I * w.H * 2
    return dict(ms=ms, distinct=float(d), bytes=float(byts))


def prefill_2k(args, lays):
    import torch
    import bit_moe_amd as bm
    import synth
    w = synth.WORKLOADS["prefill_2k"]
    x, _ = synth.make_tokens(w)
    xd = torch.from_numpy(x.view("int16")).view(torch.bfloat16).cuda()
    lay0 = lays[0]
    # prefill has no shared expert: a layer view without it
    lay = bm.Layer(w.H, w.I, w.E, w.k, *lay0.tensors[:5])
    ids = torch.empty((w.T, w.k), dtype=torch.int32, device="cuda")
    wt = torch.empty((w.T, w.k), dtype=torch.float32, device="cuda")
    y = torch.empty((w.T, w.H), dtype=torch.float32, device="cuda")
    rws = torch.empty(bm.route_workspace_bytes(lay, w.T, bm.BF16), dtype=torch.uint8, device="cuda")
    ws = torch.empty(bm.workspace_bytes(lay, w.T, bm.PREFILL), dtype=torch.uint8, device="cuda")

    def step(i):
        bm.route(lay, xd, ids=ids, w=wt, ws=rws)
        bm.ffn_prefill(lay, xd, ids, wt, y=y, ws=ws)

    ms = time_steps(step, 2, args.prefill_steps)
    gu_ms = time_dominant(step, 3)
    pairs = w.T * w.k
    flops = pairs * 3 * 2 * w.H * w.I
    gu_flops = pairs * 2 * 2 * w.H * w.I
    return dict(ms=ms, flops=flops, gu_ms=gu_ms, gu_flops=gu_flops)


def cpu_baseline(n_tokens):
    import numpy as np
    import oracle
    import synth
    w = synth.WORKLOADS["decode_b1"]
    L = synth.make_layer(w)
    x, _ = synth.make_tokens(w.with_(T=n_tokens))
    L.shared()
    t0 = time.time()
    for t in range(n_tokens):
        ids, wt = oracle.route(x[t:t + 1], L.router(), w.k)
        oracle.layer_ffn(L, x[t:t + 1], ids, wt)
    dt = time.time() - t0
    return dict(value=n_tokens / dt, unit="tokens/s", cores=oracle.max_threads(), kind="oracle",
                sample=f"{n_tokens} decode tokens (route + 8 routed experts + shared expert each) "
                       f"of the same 1-token workload, fp64, {dt:.1f}s")


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (got --gpus {args.gpus}); this build has no "
              f"multi-GPU path. Run with --gpus 1.", file=sys.stderr)
        sys.exit(2)
    import torch
    import bit_moe_amd as bm
    import synth
    bm.lib()
    assert torch.cuda.is_available(), "bench.py needs a GPU"
    w = synth.WORKLOADS["decode_b1"]
    L, lays = build_layer(w, args.copies)
    r = decode_b1(args, L, lays)
    log(f"[bench] decode_b1 {r['ms'] * 1e3:.1f} us/step, gate/up {r['gu_ms'] * 1e3:.1f} us")
    gu_bw = r["gu_bytes"] / (r["gu_ms"] * 1e-3)
    out = {
        "metric": "MoE-layer tokens/s (decode, batch 1)",
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
                   "step_hbm_GBps": r["step_bytes"] / (r["ms"] * 1e-3) / 1e9},
        "roofline": {"bound": "hbm", "kernel": "k_dec_gateup",
                     "achieved": gu_bw / 1e9, "peak": HBM_PEAK / 1e9, "unit": "GB/s",
                     "frac": gu_bw / HBM_PEAK, "traffic": None,
                     "kernel_us": r["gu_ms"] * 1e3, "algorithmic_bytes": r["gu_bytes"]},
    }
    if not args.no_extra:
        b16 = decode_b16(args, lays)
        out["decode_b16_zipf"] = {"tokens_per_s": 16 / (b16["ms"] * 1e-3), "ms_per_step": b16["ms"],
                                  "distinct_experts": b16["distinct"],
                                  "hbm_GBps": b16["bytes"] / (b16["ms"] * 1e-3) / 1e9,
                                  "hbm_frac": b16["bytes"] / (b16["ms"] * 1e-3) / HBM_PEAK,
                                  "note": "step = top-k of drawn Zipf(1.1) logits + decode FFN"}
        log(f"[bench] decode_b16 {b16['ms'] * 1e3:.1f} us/step")
        del lays[1:]
        torch.cuda.empty_cache()
        pf = prefill_2k(args, lays)
        out["prefill_2k"] = {"tokens_per_s": 2048 / (pf["ms"] * 1e-3), "ms_per_step": pf["ms"],
                             "routed_TFLOPs": pf["flops"] / (pf["ms"] * 1e-3) / 1e12,
                             "mfma_frac": pf["flops"] / (pf["ms"] * 1e-3) / BF16_PEAK,
                             "gateup_kernel_us": pf["gu_ms"] * 1e3,
                             "gateup_TFLOPs": pf["gu_flops"] / (pf["gu_ms"] * 1e-3) / 1e12,
                             "gateup_mfma_frac": pf["gu_flops"] / (pf["gu_ms"] * 1e-3) / BF16_PEAK}
        log(f"[bench] prefill_2k {pf['ms']:.2f} ms/step")
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(args.cpu_tokens)
        log(f"[bench] cpu baseline {out['cpu_baseline']['value']:.3f} tokens/s")
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
