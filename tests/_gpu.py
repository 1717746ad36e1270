"""Shared helpers of the GPU parity tests: device copies of the synthetic
layers (uploaded once per session), oracle-side margins, and the comparison
rule max|y_gpu - y_oracle| <= tol * rms(y_oracle)."""
import functools
import sys

import numpy as np
import pytest

import oracle
import synth

torch = pytest.importorskip("torch")

TOL = 2e-2          # max |err| <= 2e-2 * rms(oracle output), fp32 accumulation
MARGIN = 1e-4       # logit gap below which fp32 summation order may flip ids
# Routing weights: the weights are a softmax over the k selected logits, so
# if every GPU logit is within d of the fp64 one, every weight is within
# w (e^{2d} - 1) <= 2d (+ ~1e-6 for fp32 exp, sum and divide) of the
# oracle's: |dw| <= 2 max|dlogit| + 1e-6 (test_gpu_route checks this with the
# measured d).  Entry points that do not hand out their logits (the fused
# decode router) are held to 1e-5, i.e. d <= 4.5e-6 at H = 7168 with
# |logit| ~ 2, where fp32 accumulation of 7168 bf16 products stays.
W_TOL = 1e-5


def require_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


@functools.lru_cache(maxsize=None)
def synth_layer(w: synth.Workload):
    return synth.make_layer(w)


@functools.lru_cache(maxsize=8)
def device_layer(w: synth.Workload):
    import bit_moe_amd as bm
    L = synth_layer(w)
    say(f"[upload] {w.name} H={w.H} I={w.I} E={w.E} k={w.k} shared={w.shared} fmt={w.fmt}")
    mx = w.fmt == "mxfp4"
    lay = bm.layer_from_canonical(w.H, w.I, w.E, w.k, L.router(), L.gate_all(), L.up_all(),
                                  L.down_all(), None if mx else L.grid(), L.shared(),
                                  fmt=bm.FORMAT_MXFP4 if mx else bm.FORMAT_2BIT)
    torch.cuda.synchronize()
    return lay


def x_to_device(x: np.ndarray):
    if x.dtype == np.float32:
        return torch.from_numpy(x).cuda()
    return torch.from_numpy(x.view(np.int16)).view(torch.bfloat16).cuda()


def near_tie_tokens(logits: np.ndarray, k: int, margin: float = MARGIN) -> np.ndarray:
    s = -np.sort(-logits, axis=1)[:, :k + 1]
    gaps = s[:, :-1] - s[:, 1:]
    return np.nonzero(gaps.min(axis=1) < margin)[0]


def assert_close_rms(y_gpu: np.ndarray, y_ref: np.ndarray, tol: float = TOL, what: str = ""):
    rms = float(np.sqrt(np.mean(np.square(y_ref))))
    err = float(np.max(np.abs(y_gpu.astype(np.float64) - y_ref)))
    ratio = err / rms if rms > 0 else err
    say(f"[parity] {what} max|err|={err:.3e} rms={rms:.3e} ratio={ratio:.3e} (bar {tol})")
    assert np.all(np.isfinite(y_gpu))
    assert ratio <= tol, f"{what}: max|err|/rms = {ratio:.3e} > {tol}"
    return ratio
