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
    ap.add_argument("--prefill-steps", type=int, default=10)
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
    ap.add_argument("--prefill-only", action="store_true",
                    help="only run the 2048-token prefill step (--prefill-steps times; for counter runs)")
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
    """Average duration of the gate/up kernel, from the HIP events that its
    dispatch takes at kernel start and end (moe_set_timing_events)."""
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
    lay = bm.Layer(w.H, w.I, w.E, w.k, *lays[0].tensors[:5])
    ids = torch.empty((w.T, w.k), dtype=torch.int32, device="cuda")
    wt = torch.empty((w.T, w.k), dtype=torch.float32, device="cuda")
    y = torch.empty((w.T, w.H), dtype=torch.float32, device="cuda")
    ws = torch.empty(bm.workspace_bytes(lay, w.T, bm.PREFILL), dtype=torch.uint8, device="cuda")

    def step(i):
        bm.topk(lg, w.k, ids=ids, w=wt)
        bm.ffn_prefill(lay, xd, ids, wt, y=y, ws=ws)

    ms = time_steps(step, 1, max(2, args.prefill_steps // 4))
    rows = np.bincount(ids.cpu().numpy().ravel(), minlength=w.E)
    flops = w.T * w.k * 3 * 2 * w.H * w.I
    return dict(ms=ms, flops=flops, rows_max=int(rows.max()), rows_min=int(rows.min()))


def cpu_baseline(target_s=15.0, max_tokens=400):
    """The oracle (plain fp64 C, all host threads) on the decode workload,
    one token at a time until about target_s seconds of oracle time: routing
    and the layer per token.  Expert slabs are generated (untimed) before the
    token that first uses them."""
    import numpy as np
    import oracle
    import synth
    w = synth.WORKLOADS["decode_b1"]
    L = synth.make_layer(w)
    x, _ = synth.make_tokens(w.with_(T=max_tokens))
    grid, router, shared = L.grid(), L.router(), L.shared()
    gate, up, down = {}, {}, {}
    spent, n = 0.0, 0
    while n < max_tokens and (spent < target_s or n < 4):
        xt = x[n:n + 1]
        t0 = time.perf_counter()
        ids, wt = oracle.route(xt, router, w.k)
        spent += time.perf_counter() - t0
        for e in (int(v) for v in np.unique(ids)):
            if e not in gate:
                gate[e], up[e], down[e] = L.gate(e), L.up(e), L.down(e)
        t0 = time.perf_counter()
        oracle.moe_ffn(w.H, w.I, w.E, w.k, grid, gate, up, down, shared, xt, ids, wt)
        spent += time.perf_counter() - t0
        n += 1
    return dict(value=n / spent, unit="tokens/s", cores=oracle.max_threads(), kind="oracle",
                sample=f"{n} decode tokens of the batch-1 workload (routing + 8 routed experts + "
                       f"shared expert each, fp64), {spent:.1f} s of oracle time")


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
    for f in ("decode.hip", "common.h", "device_util.h"):
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
    first top-k, decode_b16 until the prefill step's router GEMM (the decode
    batch also runs prefill kernels, for its multi-token experts), prefill_2k
    until the 8192-token step's top-k, then prefill_8k."""
    import glob
    import sqlite3
    rows = {}
    for db in glob.glob(os.path.join(trace_dir, "**", "*.db"), recursive=True):
        c = sqlite3.connect(db)
        phase = "setup"
        for name, gx, t0, t1 in c.execute("select name, grid_x, start, end from kernels order by start"):
            if phase == "setup" and "k_dec_front" in name:
                phase = "decode_b1"
            elif phase == "decode_b1" and ("k_topk" in name or "k_dec_mid" in name):
                phase = "decode_b16"
            elif phase == "decode_b16" and "k_router_splitk" in name:
                phase = "prefill_2k"
            elif phase == "prefill_2k" and "k_topk" in name and "k_topk_sum" not in name:
                phase = "prefill_8k"
            r = rows.setdefault((phase, name, gx), [0, 0.0, float("inf"), 0.0])
            d = (t1 - t0) / 1e3
            r[0] += 1
            r[1] += d
            r[2] = min(r[2], d)
            r[3] = max(r[3], d)
    out = [f"{'phase':<11} {'calls':>6} {'avg_us':>10} {'min_us':>10} {'max_us':>10} {'grid':>10}  kernel"]
    order = {"setup": 0, "decode_b1": 1, "decode_b16": 2, "prefill_2k": 3, "prefill_8k": 4}
    for (phase, name, gx), (n, tot, mn, mx) in sorted(rows.items(), key=lambda kv: (order[kv[0][0]], -kv[1][1])):
        short = name[name.index("k_"):].split("(")[0] if "k_" in name else name.split("(")[0]
        out.append(f"{phase:<11} {n:6d} {tot / n:10.2f} {mn:10.2f} {mx:10.2f} {gx:10d}  {short}")
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
        _, lays = build_layer(synth.WORKLOADS["decode_b1"], 1)
        pf = prefill_2k(args, lays)
        log(f"[bench] prefill_2k {pf['ms']:.2f} ms/step, gate/up {pf['gu_ms'] * 1e3:.1f} us")
        return
    w = synth.WORKLOADS["decode_b1"]
    L, lays = build_layer(w, args.copies)
    r = decode_b1(args, L, lays)
    log(f"[bench] decode_b1 {r['ms'] * 1e3:.1f} us/step, gate/up {r['gu_ms'] * 1e3:.1f} us")
    gu_bw = r["gu_bytes"] / (r["gu_ms"] * 1e-3)
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
                   "step_hbm_GBps": r["step_bytes"] / (r["ms"] * 1e-3) / 1e9},
        "roofline": {"bound": "hbm", "kernel": "k_dec_gateup",
                     "achieved": gu_bw / 1e9, "peak": HBM_PEAK / 1e9, "unit": "GB/s",
                     "frac": gu_bw / HBM_PEAK, "traffic": traffic_from_profile("k_dec_gateup<1,0>"),
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
        p8 = prefill_8k_zipf(args, lays)
        out["prefill_8k_zipf"] = {"tokens_per_s": 8192 / (p8["ms"] * 1e-3), "ms_per_step": p8["ms"],
                                  "routed_TFLOPs": p8["flops"] / (p8["ms"] * 1e-3) / 1e12,
                                  "mfma_frac": p8["flops"] / (p8["ms"] * 1e-3) / BF16_PEAK,
                                  "rows_per_expert_max": p8["rows_max"], "rows_per_expert_min": p8["rows_min"],
                                  "note": "step = top-k of drawn Zipf(1.2) logits + prefill FFN"}
        log(f"[bench] prefill_8k_zipf {p8['ms']:.2f} ms/step")
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(args.cpu_seconds)
        log(f"[bench] cpu baseline {out['cpu_baseline']['value']:.3f} tokens/s")
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
