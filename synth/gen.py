"""Seeded generator of synthetic routed-MoE layers and token batches.

Everything here is *data*: packed weight bytes, bf16 weight bits, activations,
and (for the skewed workloads) router logits drawn directly.  Nothing in this
module routes a token, decodes a block or forms a product, so the oracle and
the HIP library share these inputs but none of the method's arithmetic.

Recipe (the pages publish no layer dimensions, weights or activations; these
synthetic layers stand in for DeepSeek-V4-Flash's routed experts at the model's
shapes):

* codebook ``grid``: 256 rows x 8 magnitudes, i.i.d. uniform over {1,3,5,7}.
* IQ2X superblock (66 bytes per 256 weights): the 64 bytes after the fp16
  scale are uniform random; the fp16 scale ``d`` is drawn finite and positive,
  ``d = c * U[0.5, 1.5)`` with ``c = 1 / (10.6 * sqrt(K))`` so that one output
  row has rms close to rms(x).
* Q2K superblock (84 bytes per 256 weights): the 80 bytes of scales/mins and
  2-bit quants are uniform random; ``d = c' * U[0.5, 1.5)`` and
  ``dmin = 1.5 * c' * U[0.5, 1.5)`` with ``c' = 1 / (14 * sqrt(K))``, which
  makes the weights roughly zero-mean.
* bf16 router and shared-expert weights: N(0, 0.02) rounded to bf16 (RNE).
* activations: N(0, 1), kept fp32 or rounded to bf16 (RNE).
* skewed routing: logits ``log p(rank(e)) + Gumbel(0, 1)`` with
  ``p(r) ~ (r + 1) ** -s`` over a seeded permutation of the experts; taking
  the k largest is then sampling k experts without replacement from Zipf(s).

Each (tensor, expert) and each token draws from its own counter-free stream
``PCG64(SeedSequence([seed, tensor_id, index, ...]))`` so that any single
expert or token can be regenerated alone and matches the full tensor.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, replace
from typing import Callable, Optional

import numpy as np

QK = 256                 # weights per superblock
IQ2X_BLOCK_BYTES = 66    # fp16 d + 8 groups x (4 index bytes + u32 signs/scale)
Q2K_BLOCK_BYTES = 84     # 16 scale/min bytes + 64 quant bytes + fp16 d + fp16 dmin
MXFP4_BLOCK_BYTES = 17   # E8M0 scale byte + 16 bytes of 32 E2M1 codes (32 weights)

# stream identifiers (second element of every SeedSequence entropy list)
_GRID, _ROUTER, _GATE, _UP, _DOWN, _SGATE, _SUP, _SDOWN, _X, _ZIPF = range(10)


@dataclass(frozen=True)
class Workload:
    """One synthetic layer + token batch.

    T tokens, hidden size H, expert intermediate size I, E routed experts,
    top-k routing.  ``routing`` is "computed" (logits from x and the bf16
    router) or "zipf" (logits drawn with exponent ``zipf_s``).
    """
    name: str
    T: int
    H: int
    I: int
    E: int
    k: int
    x_dtype: str          # "f32" or "bf16"
    routing: str          # "computed" or "zipf"
    zipf_s: Optional[float]
    shared: bool          # a bf16 shared expert is present
    seed: int
    mode: str             # "decode" or "prefill": the entry point it exercises
    fmt: str = "2bit"     # routed experts: "2bit" (IQ2X gate/up, Q2K down) or "mxfp4"

    def with_(self, **kw) -> "Workload":
        return replace(self, **kw)


WORKLOADS = {
    # 4 tokens, H256, I512, 8 experts, top-2, fp32 activations, seed 0
    "tiny": Workload("tiny", 4, 256, 512, 8, 2, "f32", "computed", None,
                     False, 0, "decode"),
    # one token at DeepSeek-V4-Flash MoE shapes, plus a bf16 shared expert
    "decode_b1": Workload("decode_b1", 1, 7168, 2048, 256, 8, "bf16",
                          "computed", None, True, 1, "decode"),
    # 16 concurrent decode streams, experts Zipf(1.1)-skewed
    "decode_b16_zipf": Workload("decode_b16_zipf", 16, 7168, 2048, 256, 8,
                                "bf16", "zipf", 1.1, True, 2, "decode"),
    # one 2048-token prefill chunk, uniform routing from computed logits
    "prefill_2k": Workload("prefill_2k", 2048, 7168, 2048, 256, 8, "bf16",
                           "computed", None, False, 3, "prefill"),
    # 8192-token prefill chunk, experts Zipf(1.2)-skewed
    "prefill_8k_zipf": Workload("prefill_8k_zipf", 8192, 7168, 2048, 256, 8,
                                "bf16", "zipf", 1.2, False, 4, "prefill"),
}


def _rng(*entropy: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence(list(entropy))))


def _random_bytes(rng: np.random.Generator, n: int) -> np.ndarray:
    words = rng.bit_generator.random_raw((n + 7) // 8)
    return words.view(np.uint8)[:n].copy()


def bf16_bits_from_f32(a: np.ndarray) -> np.ndarray:
    """Round float32 values to bf16 (round to nearest, ties to even); return the
    16-bit patterns.  Inputs here are finite, so no NaN handling is needed."""
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32).astype(np.uint64)
    r = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return r.astype(np.uint16)


def f32_from_bf16_bits(b: np.ndarray) -> np.ndarray:
    """Widen bf16 bit patterns to float32 (exact)."""
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def _fp16_bytes(v: np.ndarray) -> np.ndarray:
    h = np.asarray(v, dtype=np.float16)
    assert np.all(np.isfinite(h)) and np.all(h > 0)
    return h.view(np.uint8).reshape(-1, 2)


def iq2x_slab(seed: int, tensor: int, e: int, N: int, K: int) -> np.ndarray:
    """Canonical IQ2X blocks of one expert's [N, K] projection:
    uint8 [N * K/256, 66], block (n, kb) at row n*(K/256)+kb."""
    nb = N * (K // QK)
    rng = _rng(seed, tensor, e)
    raw = _random_bytes(rng, nb * IQ2X_BLOCK_BYTES).reshape(nb, IQ2X_BLOCK_BYTES)
    c = 1.0 / (10.6 * math.sqrt(K))
    raw[:, 0:2] = _fp16_bytes(c * rng.uniform(0.5, 1.5, nb))
    return raw


def mxfp4_slab(seed: int, tensor: int, e: int, N: int, K: int) -> np.ndarray:
    """Canonical MXFP4 blocks of one expert's [N, K] projection: uint8
    [N * K/32, 17], block (n, kb) at row n*(K/32)+kb.  The 16 element bytes
    are uniform random; the E8M0 scale byte X is drawn around
    127 + log2(1 / (2.93 sqrt(K))), +-1 (the rms of a uniform random E2M1
    code is 2.93), so that one output row has rms close to rms(x)."""
    nb = N * (K // 32)
    rng = _rng(seed, tensor, e)
    raw = _random_bytes(rng, nb * MXFP4_BLOCK_BYTES).reshape(nb, MXFP4_BLOCK_BYTES)
    centre = 127 + int(round(math.log2(1.0 / (2.93 * math.sqrt(K)))))
    raw[:, 0] = centre + rng.integers(-1, 2, nb)
    return raw


def q2k_slab(seed: int, tensor: int, e: int, N: int, K: int) -> np.ndarray:
    """Canonical Q2K blocks of one expert's [N, K] projection:
    uint8 [N * K/256, 84]."""
    nb = N * (K // QK)
    rng = _rng(seed, tensor, e)
    raw = _random_bytes(rng, nb * Q2K_BLOCK_BYTES).reshape(nb, Q2K_BLOCK_BYTES)
    c = 1.0 / (14.0 * math.sqrt(K))
    raw[:, 80:82] = _fp16_bytes(c * rng.uniform(0.5, 1.5, nb))
    raw[:, 82:84] = _fp16_bytes(1.5 * c * rng.uniform(0.5, 1.5, nb))
    return raw


def _bf16_normal(seed: int, tensor: int, shape, std: float) -> np.ndarray:
    rng = _rng(seed, tensor)
    return bf16_bits_from_f32((rng.standard_normal(shape) * std).astype(np.float32))


class Layer:
    """Lazily generated weights of one synthetic layer (canonical layouts).

    Per-expert slabs come from independent streams, so ``gate(e)`` equals
    rows ``[e*I*H/256, (e+1)*I*H/256)`` of ``gate_all()``.
    """

    def __init__(self, w: Workload):
        self.w = w
        self._cache = {}

    def _memo(self, key, fn):
        if key not in self._cache:
            self._cache[key] = fn()
        return self._cache[key]

    # codebook: 256 x 8 magnitudes in {1,3,5,7}
    def grid(self) -> np.ndarray:
        def mk():
            rng = _rng(self.w.seed, _GRID)
            return (2 * rng.integers(0, 4, size=(256, 8)) + 1).astype(np.uint8)
        return self._memo("grid", mk)

    def router(self) -> np.ndarray:
        """bf16 bits [E, H]."""
        return self._memo("router", lambda: _bf16_normal(
            self.w.seed, _ROUTER, (self.w.E, self.w.H), 0.02))

    def gate(self, e: int) -> np.ndarray:
        if self.w.fmt == "mxfp4":
            return mxfp4_slab(self.w.seed, _GATE, e, self.w.I, self.w.H)
        return iq2x_slab(self.w.seed, _GATE, e, self.w.I, self.w.H)

    def up(self, e: int) -> np.ndarray:
        if self.w.fmt == "mxfp4":
            return mxfp4_slab(self.w.seed, _UP, e, self.w.I, self.w.H)
        return iq2x_slab(self.w.seed, _UP, e, self.w.I, self.w.H)

    def down(self, e: int) -> np.ndarray:
        if self.w.fmt == "mxfp4":
            return mxfp4_slab(self.w.seed, _DOWN, e, self.w.H, self.w.I)
        return q2k_slab(self.w.seed, _DOWN, e, self.w.H, self.w.I)

    def _all(self, fn) -> np.ndarray:
        return np.concatenate([fn(e) for e in range(self.w.E)], axis=0)

    def gate_all(self) -> np.ndarray:
        return self._all(self.gate)

    def up_all(self) -> np.ndarray:
        return self._all(self.up)

    def down_all(self) -> np.ndarray:
        return self._all(self.down)

    def shared(self):
        """(gate [I,H], up [I,H], down [H,I]) bf16 bits, or None."""
        if not self.w.shared:
            return None

        def mk():
            w = self.w
            return (_bf16_normal(w.seed, _SGATE, (w.I, w.H), 0.02),
                    _bf16_normal(w.seed, _SUP, (w.I, w.H), 0.02),
                    _bf16_normal(w.seed, _SDOWN, (w.H, w.I), 0.02))
        return self._memo("shared", mk)


def make_layer(w: Workload) -> Layer:
    return Layer(w)


def token_row(w: Workload, t: int, attempt: int = 0) -> np.ndarray:
    """Activation row of token t: float32 [H] for "f32", bf16 bits for "bf16"."""
    rng = _rng(w.seed, _X, t, attempt)
    v = rng.standard_normal(w.H).astype(np.float32)
    return v if w.x_dtype == "f32" else bf16_bits_from_f32(v)


def make_tokens(w: Workload, accept: Optional[Callable[[int, np.ndarray], bool]] = None,
                max_attempts: int = 64, T: Optional[int] = None):
    """Token batch x [T, H] (float32, or uint16 bf16 bits).

    ``accept(t, row)`` may reject a drawn row (the caller uses it to keep
    router logits margin-separated); a rejected token is redrawn from the
    next attempt of its own stream.  Returns (x, attempts)."""
    T = w.T if T is None else T
    rows, attempts = [], np.zeros(T, dtype=np.int32)
    for t in range(T):
        for a in range(max_attempts):
            r = token_row(w, t, a)
            if accept is None or accept(t, r):
                break
        else:
            raise RuntimeError(f"token {t}: no acceptable draw in {max_attempts}")
        rows.append(r)
        attempts[t] = a
    return np.stack(rows), attempts


def zipf_logits(w: Workload, T: Optional[int] = None) -> np.ndarray:
    """Drawn router logits float32 [T, E] for the skewed workloads."""
    T = w.T if T is None else T
    assert w.zipf_s is not None
    rng = _rng(w.seed, _ZIPF)
    rank_of = rng.permutation(w.E)                  # rank of expert e
    logp = -w.zipf_s * np.log(rank_of + 1.0)        # unnormalised log p
    g = rng.gumbel(size=(T, w.E))
    return (logp[None, :] + g).astype(np.float32)
