"""Seeded synthetic inputs for weight-quantization tuning (shared by the
oracle-based tests, the GPU tests and the benchmark).

This module draws random numbers and casts them to the storage dtype; it holds
none of the quantization method's arithmetic.  Every workload the pages
describe (trained LLM weights and real calibration text, e.g. 128 samples x
2048 tokens in the AutoRound blog's preset table, "Second Gate" section of
"Low-Bit Quantization in Practice with vLLM") is replaced by this recipe:

* weights W[N, K] ~ N(0, 0.02^2); exactly round(0.001 * N * K) distinct
  positions, drawn uniformly without replacement, are multiplied by 20
  (sign kept) -- the outliers the pages' error taxonomy is about;
* calibration activations X[S, T, K] ~ N(0, 1); c distinct channels drawn
  uniformly are multiplied by 50 for every token;
* a minibatch schedule [iters, B] of sample ids: one fresh permutation of
  the S samples per epoch, cut into consecutive chunks of B;
* bf16 storage is the round-to-nearest-even cast of the fp32 draw (torch's
  CPU cast), so both sides of a comparison see identical values.

All draws come from numpy.random.default_rng(seed) in the fixed order
W, X, schedule.

Block workloads (the gated MLP of a Llama-style decoder, tuned block-wise):
the three weights (gate [F, H], up [F, H], down [H, F]) follow the weight
recipe, drawn in that order; the pool is the block's input, i.e. N(0, 1)
tokens passed through an RMS normalization with unit weight and eps 1e-5
(each token row divided by sqrt(mean(x^2) + eps)); then the schedule.

Decoder workloads (a whole Llama-style decoder block): the seven weights q,
k, v, o, gate, up, down follow the weight recipe, drawn in that order; then
the two RMSNorm weights [H] ~ U(0.8, 1.2); the pool is the block's input
(the residual stream) drawn with the calibration recipe (N(0, 1) with c
outlier channels x50); then the schedule.  Storage is bf16 (norm weights
fp32).
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np

__all__ = [
    "LayerWorkload",
    "make_weight",
    "make_calibration",
    "make_schedule",
    "make_layer_workload",
    "WORKLOADS",
    "BlockWorkload",
    "BLOCK_WORKLOADS",
    "make_block_workload",
    "to_bf16_values",
    "DecoderWorkload",
    "DECODER_WORKLOADS",
    "make_decoder_workload",
]


def to_bf16_values(a: np.ndarray) -> np.ndarray:
    """Round an fp32 array to the nearest bf16 value (ties to even) and return
    it widened back to fp32; the result is exactly representable in bf16."""
    import torch

    t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32))
    return t.to(torch.bfloat16).to(torch.float32).numpy()


def make_weight(rng: np.random.Generator, n: int, k: int, std: float = 0.02,
                outlier_frac: float = 0.001, outlier_scale: float = 20.0) -> np.ndarray:
    w = rng.standard_normal((n, k), dtype=np.float32) * np.float32(std)
    n_out = int(round(outlier_frac * n * k))
    if n_out > 0:
        idx = rng.choice(n * k, size=n_out, replace=False)
        w.reshape(-1)[idx] *= np.float32(outlier_scale)
    return w


def make_calibration(rng: np.random.Generator, s: int, t: int, k: int,
                     n_outlier_channels: int, outlier_scale: float = 50.0) -> np.ndarray:
    x = rng.standard_normal((s, t, k), dtype=np.float32)
    if n_outlier_channels > 0:
        ch = rng.choice(k, size=n_outlier_channels, replace=False)
        x[:, :, ch] *= np.float32(outlier_scale)
    return x


def make_schedule(rng: np.random.Generator, s: int, b: int, iters: int) -> np.ndarray:
    """[iters, b] int32 sample ids; per-epoch permutation cut into chunks of b.
    When b == s every row is the whole pool in order (full batch)."""
    if b == s:
        return np.tile(np.arange(s, dtype=np.int32), (iters, 1))
    rows = []
    perm = rng.permutation(s).astype(np.int32)
    pos = 0
    for _ in range(iters):
        if pos + b > s:
            perm = rng.permutation(s).astype(np.int32)
            pos = 0
        rows.append(perm[pos:pos + b])
        pos += b
    return np.stack(rows).astype(np.int32)


@dataclass
class LayerWorkload:
    """One single-linear-layer tuning problem."""

    name: str
    n: int
    k: int
    s: int                   # calibration samples in the pool
    t: int                   # tokens per sample
    b: int                   # samples per step
    bits: int
    group: int
    iters: int
    lr: float
    dtype: str               # storage dtype of W and X: "f32" or "bf16"
    n_outlier_channels: int
    seed: int
    W: np.ndarray = field(repr=False, default=None)       # fp32 values [n, k]
    X: np.ndarray = field(repr=False, default=None)       # fp32 values [s, t, k]
    schedule: np.ndarray = field(repr=False, default=None)  # int32 [iters, b]


# Single-linear workloads.  "linear256_g32" is the small validation layer;
# "linear4096_g128" is the 4096x4096 int4 g128 layer with a 128 x 256-token
# pool and 8-sample (2048-token) minibatches.
WORKLOADS = {
    "linear256_g32": dict(n=256, k=256, s=1, t=64, b=1, bits=4, group=32, iters=20,
                          lr=0.005, dtype="f32", n_outlier_channels=4, seed=0),
    "linear4096_g128": dict(n=4096, k=4096, s=128, t=256, b=8, bits=4, group=128,
                            iters=200, lr=0.005, dtype="bf16", n_outlier_channels=8, seed=1),
}


def make_layer_workload(name: str, **overrides) -> LayerWorkload:
    """Build a workload by name; keyword overrides (e.g. n=512, s=4) shrink it
    for tests while keeping the recipe.  Draw order: W, X, schedule."""
    cfg = dict(WORKLOADS[name])
    cfg.update(overrides)
    wl = LayerWorkload(name=name, **cfg)
    rng = np.random.default_rng(wl.seed)
    w = make_weight(rng, wl.n, wl.k)
    x = make_calibration(rng, wl.s, wl.t, wl.k, wl.n_outlier_channels)
    sched = make_schedule(rng, wl.s, wl.b, wl.iters)
    if wl.dtype == "bf16":
        w = to_bf16_values(w)
        x = to_bf16_values(x)
    elif wl.dtype != "f32":
        raise ValueError(f"unknown dtype {wl.dtype}")
    wl.W, wl.X, wl.schedule = w, x, sched
    return wl


@dataclass
class BlockWorkload:
    """One SwiGLU MLP block tuning problem (hidden h, intermediate f)."""

    name: str
    h: int
    f: int
    s: int
    t: int
    b: int
    bits: int
    group: int
    iters: int
    lr: float
    dtype: str
    seed: int
    norm_eps: float = 1e-5
    Wg: np.ndarray = field(repr=False, default=None)      # [f, h]
    Wu: np.ndarray = field(repr=False, default=None)      # [f, h]
    Wd: np.ndarray = field(repr=False, default=None)      # [h, f]
    X: np.ndarray = field(repr=False, default=None)       # [s, t, h]
    schedule: np.ndarray = field(repr=False, default=None)


# "mlp4096_11008_g128": the Llama-7B-shaped MLP (hidden 4096, intermediate
# 11008), int4 g128, the same pool and minibatch sizes as the layer workload.
BLOCK_WORKLOADS = {
    "mlp4096_11008_g128": dict(h=4096, f=11008, s=128, t=256, b=8, bits=4, group=128, iters=200, lr=0.005,
                               dtype="bf16", seed=2),
}


def make_block_workload(name: str, **overrides) -> BlockWorkload:
    """Build a block workload by name (keyword overrides shrink it for tests).
    Draw order: gate, up, down, pool, schedule."""
    cfg = dict(BLOCK_WORKLOADS[name])
    cfg.update(overrides)
    wl = BlockWorkload(name=name, **cfg)
    rng = np.random.default_rng(wl.seed)
    wg = make_weight(rng, wl.f, wl.h)
    wu = make_weight(rng, wl.f, wl.h)
    wd = make_weight(rng, wl.h, wl.f)
    x = rng.standard_normal((wl.s, wl.t, wl.h), dtype=np.float32)
    x /= np.sqrt(np.mean(x * x, axis=2, keepdims=True) + np.float32(wl.norm_eps))
    sched = make_schedule(rng, wl.s, wl.b, wl.iters)
    if wl.dtype == "bf16":
        wg, wu, wd, x = (to_bf16_values(a) for a in (wg, wu, wd, x))
    elif wl.dtype != "f32":
        raise ValueError(f"unknown dtype {wl.dtype}")
    wl.Wg, wl.Wu, wl.Wd, wl.X, wl.schedule = wg, wu, wd, x.astype(np.float32), sched
    return wl


@dataclass
class DecoderWorkload:
    """One Llama-style decoder block tuning problem."""

    name: str
    h: int
    f: int
    heads: int
    kv_heads: int
    head_dim: int
    s: int
    t: int
    b: int
    bits: int
    group: int
    iters: int
    lr: float
    seed: int
    n_outlier_channels: int = 8
    norm_eps: float = 1e-5
    rope_theta: float = 10000.0
    W: dict = field(repr=False, default=None)             # name -> fp32 values [N, K]
    w1: np.ndarray = field(repr=False, default=None)      # [h] fp32
    w2: np.ndarray = field(repr=False, default=None)
    X: np.ndarray = field(repr=False, default=None)       # [s, t, h] fp32 values of bf16
    schedule: np.ndarray = field(repr=False, default=None)

    def shapes(self):
        nq, nkv = self.heads * self.head_dim, self.kv_heads * self.head_dim
        return {"q": (nq, self.h), "k": (nkv, self.h), "v": (nkv, self.h), "o": (self.h, nq),
                "gate": (self.f, self.h), "up": (self.f, self.h), "down": (self.h, self.f)}

    def cfg(self):
        """Block description in the decoder oracle's form."""
        return dict(H=self.h, nq=self.heads, nkv=self.kv_heads, d=self.head_dim, F=self.f, T=self.t,
                    eps=self.norm_eps, theta=self.rope_theta, w1=self.w1, w2=self.w2)


# "llama7b_decoder_g128": Llama-7B-shaped block (hidden 4096, 32 heads x 128,
# FFN 11008), 256-token samples, int4 g128, 8 samples per step.
# "llama70b_decoder_g32": 70B-shaped block (hidden 8192, 64 query / 8 KV
# heads x 128, FFN 28672), int4 g32, 4 samples per step.
DECODER_WORKLOADS = {
    "llama7b_decoder_g128": dict(h=4096, f=11008, heads=32, kv_heads=32, head_dim=128, s=128, t=256, b=8,
                                 bits=4, group=128, iters=200, lr=0.005, seed=3),
    "llama70b_decoder_g32": dict(h=8192, f=28672, heads=64, kv_heads=8, head_dim=128, s=128, t=256, b=4,
                                 bits=4, group=32, iters=200, lr=0.005, seed=4),
}


def make_decoder_workload(name: str, **overrides) -> DecoderWorkload:
    """Build a decoder workload by name (keyword overrides shrink it for
    tests).  Draw order: q, k, v, o, gate, up, down, w1, w2, pool, schedule."""
    cfg = dict(DECODER_WORKLOADS[name])
    cfg.update(overrides)
    wl = DecoderWorkload(name=name, **cfg)
    rng = np.random.default_rng(wl.seed)
    wl.W = {nm: to_bf16_values(make_weight(rng, n, k)) for nm, (n, k) in wl.shapes().items()}
    wl.w1 = rng.uniform(0.8, 1.2, wl.h).astype(np.float32)
    wl.w2 = rng.uniform(0.8, 1.2, wl.h).astype(np.float32)
    wl.X = to_bf16_values(make_calibration(rng, wl.s, wl.t, wl.h, wl.n_outlier_channels))
    wl.schedule = make_schedule(rng, wl.s, wl.b, wl.iters)
    return wl
