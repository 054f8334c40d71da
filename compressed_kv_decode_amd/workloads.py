"""Seeded synthetic inputs for the compressed-KV decode path.

This module only draws random data of the shapes and distributions of the
five workloads below.  It holds none of the method's arithmetic (no rotation,
quantisation, sketch or attention) and imports neither the HIP binding nor
the oracle, so that both sides can take their inputs from it.

Workloads (sizes stated in full; the model names describe attention shapes,
no weights are involved):

* ``tiny``: 1 sequence, 1 layer, 4 query = 4 kv heads, head_dim 64, window
  256, prefill 1024 (256 hot + 768 cold) in F3, K/V ~ N(0,1) with 4 outlier
  channels x8 per (layer, kv head), drawn independently for K and V;
  8 decode steps; promotion off.
* ``tinyllama``: TinyLlama-1.1B-shaped attention: 22 layers, 32 q / 4 kv
  heads, head_dim 64, batch 1, window 512, prefill 1536 (512 hot + 1024
  cold) in F3, K/V ~ N(0,1) times per-channel LogNormal(0, 0.5) scales per
  (layer, kv head); 50 decode steps with eviction every step and promotion
  (threshold 0.15, sticky 3) driven by two planted heavy hitters per layer.
* ``llama8b``: Llama-3.1-8B-shaped: 32 layers, 32 q / 8 kv heads, head_dim
  128, batch 8, context 32768 (512 hot + rest cold), F3 or F4, K/V Gaussian
  with 1% of each layer's kv channels (10 of 1024) scaled x10; 64 decode
  steps.
* ``long``: 1 sequence, 1 layer, 32 q / 8 kv, head_dim 128, 131072-token
  prefill in one append (130560 cold in F2.5), 32 decode steps, one needle:
  a key aligned with every query of its group, planted at a random depth.
* ``ragged``: Mistral-7B-shaped (32 q / 8 kv, head_dim 128), 64 sequences
  with contexts LogNormal(ln 4096, ln 16 / 4) rounded and clipped to
  [1024, 16384], window 512, 32 layers alternating F3 (even) / F4 (odd),
  128 decode steps with eviction and promotion, planted heavy hitters.

Queries are N(0, I) in fp16 unless a heavy hitter or the needle aligns them.
All draws come from numpy's default_rng seeded by SeedSequence([seed,
workload id, purpose, layer, sequence, step]); values are rounded to fp16
(round-to-nearest-even) before anyone sees them.
"""

from dataclasses import dataclass, field, replace
from typing import Optional, Tuple

import numpy as np

# format triples (r_bits, theta_bits, qjl_m)
F3 = (2, 3, 32)
F4 = (3, 4, 64)
F25 = (2, 2, 64)

_PURPOSE = dict(scale=1, prefill_k=2, prefill_v=3, step_k=4, step_v=5, query=6,
                hitters=7, needle=8, lengths=9, outlier=10)


@dataclass(frozen=True)
class Workload:
    name: str
    wid: int
    n_seq: int
    n_layers: int
    n_q_heads: int
    n_kv_heads: int
    head_dim: int
    window: int
    prefill: Tuple[int, ...]  # per sequence
    formats: Tuple[Tuple[int, int, int], ...]  # per layer
    steps: int
    tau: float = 2.0  # > 1 disables promotion
    sticky: int = 3
    seed: int = 0
    outlier_channels: int = 0  # per (layer, kv head), K and V independently
    outlier_frac_layer: float = 0.0  # fraction of the layer's H_kv * d channels
    outlier_scale: float = 1.0
    lognormal_sigma: float = 0.0  # per-channel LogNormal(0, sigma) scales
    heavy_hitters: int = 0  # per (sequence, layer)
    needle: bool = False
    v_qjl: bool = True

    @property
    def group(self) -> int:
        return self.n_q_heads // self.n_kv_heads

    def max_context(self) -> int:
        return max(self.prefill) + self.steps

    def fmt(self, layer: int):
        return self.formats[layer]

    def with_(self, **kw) -> "Workload":
        return replace(self, **kw)


def _ragged_lengths(seed: int, n: int) -> Tuple[int, ...]:
    rng = np.random.default_rng(np.random.SeedSequence([seed, 5, _PURPOSE["lengths"]]))
    x = rng.lognormal(mean=np.log(4096.0), sigma=np.log(16.0) / 4.0, size=n)
    return tuple(int(v) for v in np.clip(np.rint(x), 1024, 16384))


def make(name: str, seed: int = 0, fmt: Optional[Tuple[int, int, int]] = None) -> Workload:
    """The named workload at full size."""
    if name == "tiny":
        return Workload("tiny", 1, 1, 1, 4, 4, 64, 256, (1024,), (F3,), 8, seed=seed,
                        outlier_channels=4, outlier_scale=8.0)
    if name == "tinyllama":
        return Workload("tinyllama", 2, 1, 22, 32, 4, 64, 512, (1536,), (F3,) * 22, 50,
                        tau=0.15, sticky=3, seed=seed, lognormal_sigma=0.5, heavy_hitters=2)
    if name == "llama8b":
        f = fmt or F3
        return Workload("llama8b", 3, 8, 32, 32, 8, 128, 512, (32768,) * 8, (f,) * 32, 64,
                        seed=seed, outlier_frac_layer=0.01, outlier_scale=10.0)
    if name == "long":
        return Workload("long", 4, 1, 1, 32, 8, 128, 512, (131072,), (F25,), 32,
                        seed=seed, needle=True)
    if name == "ragged":
        return Workload("ragged", 5, 64, 32, 32, 8, 128, 512, _ragged_lengths(seed, 64),
                        tuple(F3 if l % 2 == 0 else F4 for l in range(32)), 128,
                        tau=0.15, sticky=3, seed=seed, heavy_hitters=2)
    raise KeyError(name)


def _rng(w: Workload, purpose: str, *ids) -> np.random.Generator:
    return np.random.default_rng(np.random.SeedSequence([w.seed, w.wid, _PURPOSE[purpose], *ids]))


def channel_scales(w: Workload, layer: int, which: str) -> np.ndarray:
    """Per (kv head, channel) multipliers [H_kv, d] of K ('k') or V ('v')."""
    h, d = w.n_kv_heads, w.head_dim
    sc = np.ones((h, d))
    tag = 0 if which == "k" else 1
    if w.outlier_channels:
        rng = _rng(w, "outlier", layer, tag)
        for kv in range(h):
            ch = rng.choice(d, size=w.outlier_channels, replace=False)
            sc[kv, ch] = w.outlier_scale
    if w.outlier_frac_layer:
        rng = _rng(w, "outlier", layer, tag)
        n = int(round(w.outlier_frac_layer * h * d))
        flat = rng.choice(h * d, size=n, replace=False)
        sc.reshape(-1)[flat] = w.outlier_scale
    if w.lognormal_sigma:
        rng = _rng(w, "scale", layer, tag)
        sc = sc * rng.lognormal(0.0, w.lognormal_sigma, size=(h, d))
    return sc


def _kv_draw(w: Workload, purpose: str, layer: int, seq: int, n: int, which: str, *extra) -> np.ndarray:
    rng = _rng(w, purpose, layer, seq, *extra)
    x = rng.standard_normal((n, w.n_kv_heads, w.head_dim)) * channel_scales(w, layer, which)[None]
    return x.astype(np.float16)


def hitters(w: Workload, layer: int, seq: int):
    """Planted heavy hitters of a (layer, sequence): list of
    (token index, kv head, on-steps).  Their tokens sit in the part of the
    prefill that starts cold; queries of the kv head's group align with the
    hitter's key on the on-steps (runs of 1, 2, 3 and 5 steps)."""
    if not w.heavy_hitters:
        return []
    n_cold0 = w.prefill[seq] - w.window
    rng = _rng(w, "hitters", layer, seq)
    toks = rng.choice(n_cold0, size=w.heavy_hitters, replace=False)
    out = []
    for i, t in enumerate(toks):
        base = 1 + 20 * i
        on = []
        s = base
        for run in (1, 2, 3, 5):
            on.extend(range(s, s + run))
            s += run + 2
        on = [x for x in on if x < w.steps]
        out.append((int(t), i % w.n_kv_heads, tuple(on)))
    return out


def needle(w: Workload, seq: int = 0):
    """(token index, unit directions [H_kv, d], key scale) of the needle.

    The needle's key in kv head g is kappa * u_g; every query of group g is
    sqrt(d) * u_g + 0.25 * N(0, I).  kappa = ln(49 N e^0.53) makes the
    needle's logit exceed the log of the summed weight of the N other keys
    (logits ~ N(0, 1.06)) by ln 49, i.e. about 0.98 of the exact attention
    mass (a closed-form choice; the tests measure the actual mass).
    """
    rng = _rng(w, "needle", 0, seq)
    n_cold0 = w.prefill[seq] - w.window
    tok = int(rng.integers(0, n_cold0))
    u = rng.standard_normal((w.n_kv_heads, w.head_dim))
    u /= np.linalg.norm(u, axis=1, keepdims=True)
    kappa = float(np.log(49.0 * w.prefill[seq] * np.exp(0.53)))
    return tok, u, kappa


def prefill_kv(w: Workload, layer: int, seq: int, start: int = 0, stop: Optional[int] = None):
    """Prefill K and V tokens [start, stop) of (layer, seq): fp16 [n, H_kv, d]."""
    n = w.prefill[seq]
    stop = n if stop is None else stop
    k = _kv_draw(w, "prefill_k", layer, seq, n, "k")
    v = _kv_draw(w, "prefill_v", layer, seq, n, "v")
    if w.needle:
        tok, u, kappa = needle(w, seq)
        k[tok] = (kappa * u).astype(np.float16)
    return k[start:stop], v[start:stop]


def step_kv(w: Workload, layer: int, seq: int, step: int):
    """The token appended at decode step ``step`` (0-based): fp16 [1, H_kv, d]."""
    k = _kv_draw(w, "step_k", layer, seq, 1, "k", step)
    v = _kv_draw(w, "step_v", layer, seq, 1, "v", step)
    return k, v


def query(w: Workload, layer: int, seq: int, step: int) -> np.ndarray:
    """Decode-step queries fp16 [H_q, d]."""
    rng = _rng(w, "query", layer, seq, step)
    g = w.group
    if w.needle:
        _, u, _ = needle(w, seq)
        q = np.sqrt(w.head_dim) * np.repeat(u, g, axis=0) + 0.25 * rng.standard_normal((w.n_q_heads, w.head_dim))
        return q.astype(np.float16)
    q = rng.standard_normal((w.n_q_heads, w.head_dim))
    if w.heavy_hitters:
        k_all, _ = prefill_kv(w, layer, seq)
        n = w.prefill[seq]
        for tok, kv, on in hitters(w, layer, seq):
            if step in on:
                kk = k_all[tok, kv].astype(np.float64)
                # hitter logit about ln(n) + 2 above a typical key's
                kap = (np.log(n) + 2.0) * np.sqrt(w.head_dim) / np.linalg.norm(kk)
                q[kv * g:(kv + 1) * g] += kap * kk / np.linalg.norm(kk)
    return q.astype(np.float16)
