"""Seeded synthetic inputs for the wave index: keys, values and decode queries.

This module serves the tests, the bench and the CPU oracle alike. It holds no
part of the wave-index arithmetic (no clustering, scoring, selection or
attention); it only draws the inputs and formats them as bf16 bit patterns.

The workloads stand in for the long-context benchmarks (RULER,
Needle-in-a-Haystack on Llama3 / Qwen2.5) that the RetroInfer summaries
evaluate on (gist.science summaries, section 4 "Results"): head shapes of those
models, contexts from 4K to 1M tokens, and a retrieval-like structure. Keys
follow a piecewise-constant topic sequence, rotated by RoPE so that nearby
positions stay similar (the locality that the summaries' segmented clustering
relies on, gist.science/zh section 2A). The query is aimed at one topic present
in the context, plus a fixed per-head shift that makes it out-of-distribution
with respect to the keys (the query/key distribution gap described on the
RetrievalAttention abstract page).

Recipe, per batch element b, layer l, KV head g, query head h:
  * topics: z_t for t in [0, L0 + steps), piece lengths ~ Geometric(1/mean),
    each piece's topic uniform on {0..63}; shared by all layers and heads of b.
  * centres: mu_0..63 ~ N(0, I_d) per (l, g).
  * keys: k_t = RoPE(t) (mu_{z_t} + 0.5 eps_t), eps_t ~ N(0, I).
  * values: v_t ~ N(0, I).
  * query at step s (position p = L0 + s): q = RoPE(p) (0.8 mu_{z*} + xi + delta_h)
    with xi ~ N(0, I) fresh per (b, l, h, s), delta_h ~ N(0, 0.5 I) fixed per
    (l, h), z* = z_{t*} with t* uniform over the indexed positions, drawn per
    (b, l, g, s).
  * training queries of KV head g (the prefill queries an attention-aware vector index
    learns the query distribution from): at each of the last n_pos prefill positions
    p = L0 - n_pos + i, one query per head h of the group, q = RoPE(p) (0.8 mu_{z*} + xi
    + delta_h) as above (delta_h the same fixed shift), with z* = z_{t*}, t* uniform over
    the indexed positions, drawn per (b, l, g, i); ordered i-major, head-minor.
  * RoPE: half-split pairs (i, i + d/2), theta_i = base^(-2i/d), angles in fp64.
  * numbers are drawn in fp32/fp64 with numpy PCG64 seeded by
    SeedSequence(seed, spawn_key=(b, l, head, kind)) and rounded to bf16
    (round-to-nearest-even, through fp32).
"""
from __future__ import annotations

import math
import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, field, replace

import numpy as np

__all__ = ["Workload", "WORKLOADS", "LayerInputs", "generate_layer", "training_queries",
           "f32_to_bf16_bits", "bf16_bits_to_f32"]

# spawn-key "kind" tags, one per independent random stream
_TOPIC, _CENTRES, _KEYNOISE, _VALUES, _QTARGET, _QNOISE, _QSHIFT, _TTARGET, _TNOISE = range(9)
N_TOPICS = 64


@dataclass(frozen=True)
class Workload:
    """One synthetic workload: model head shapes, context and index parameters."""
    name: str
    batch: int
    n_layers: int
    n_q_heads: int
    n_kv_heads: int
    head_dim: int
    context: int            # L0: prefilled, indexed length
    segment_size: int       # S
    cluster_size: int       # average cluster size; clusters per segment = S / cluster_size
    n_iters: int            # k-means assignment passes
    n_sink: int
    n_recent: int
    budget: float           # retrieval budget as a fraction of the clusters
    steps: int              # decode steps
    topic_mean: int = 256   # mean topic-piece length
    rope_base: float = 5e5
    seed: int = 1000
    notes: str = field(default="", compare=False)

    @property
    def group(self) -> int:
        return self.n_q_heads // self.n_kv_heads

    @property
    def clusters_per_segment(self) -> int:
        return self.segment_size // self.cluster_size

    @property
    def n_segments(self) -> int:
        return -(-self.context // self.segment_size)

    @property
    def n_clusters(self) -> int:
        return self.n_segments * self.clusters_per_segment

    @property
    def n_retrieve(self) -> int:
        # integer retrieval budget: ceil(budget * C), with a guard against fp noise
        return int(math.ceil(self.budget * self.n_clusters - 1e-9))

    @property
    def capacity(self) -> int:
        return self.context + self.steps

    def with_(self, **kw) -> "Workload":
        return replace(self, **kw)


WORKLOADS = {
    # 1 layer, B1, 4K context, one segment of 256 clusters, 5 iterations, 4 + 64 steady, 2 %.
    "tiny": Workload("tiny", batch=1, n_layers=1, n_q_heads=32, n_kv_heads=8, head_dim=128,
                     context=4096, segment_size=4096, cluster_size=16, n_iters=5, n_sink=4,
                     n_recent=64, budget=0.02, steps=16, seed=1001),
    # Llama-3-8B-shaped single layer at 128K: 8192-token segments, cluster size 16, 10 iterations.
    "llama128k": Workload("llama128k", batch=1, n_layers=1, n_q_heads=32, n_kv_heads=8,
                          head_dim=128, context=131072, segment_size=8192, cluster_size=16,
                          n_iters=10, n_sink=4, n_recent=512, budget=0.018, steps=64, seed=1002),
    # Llama-3-8B-shaped 32-layer stack, batch 8 at 122 880 context.
    "llama122k_b8": Workload("llama122k_b8", batch=8, n_layers=32, n_q_heads=32, n_kv_heads=8,
                             head_dim=128, context=122880, segment_size=8192, cluster_size=16,
                             n_iters=10, n_sink=4, n_recent=512, budget=0.018, steps=64,
                             seed=1003),
    # 1M-token context, 32 layers, batch 1.
    "llama1m": Workload("llama1m", batch=1, n_layers=32, n_q_heads=32, n_kv_heads=8,
                        head_dim=128, context=1048576, segment_size=8192, cluster_size=16,
                        n_iters=10, n_sink=4, n_recent=1024, budget=0.018, steps=64, seed=1004),
    # Qwen2.5-7B-shaped: 28 q / 4 KV heads (G = 7), batch 4, 256K, short topic pieces.
    "qwen256k": Workload("qwen256k", batch=4, n_layers=28, n_q_heads=28, n_kv_heads=4,
                         head_dim=128, context=262144, segment_size=8192, cluster_size=16,
                         n_iters=10, n_sink=4, n_recent=512, budget=0.018, steps=64,
                         topic_mean=64, seed=1005),
}


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """float32 -> bf16 bit pattern (uint16), round to nearest even (finite inputs)."""
    b = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    b = b + (np.uint32(0x7FFF) + ((b >> np.uint32(16)) & np.uint32(1)))
    return (b >> np.uint32(16)).astype(np.uint16)


def bf16_bits_to_f32(u: np.ndarray) -> np.ndarray:
    """bf16 bit pattern (uint16) -> float32 (exact)."""
    return (np.asarray(u, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def _rng(w: Workload, b: int, layer: int, head: int, kind: int) -> np.random.Generator:
    ss = np.random.SeedSequence(w.seed, spawn_key=(b, layer, head, kind))
    return np.random.Generator(np.random.PCG64(ss))


def _rope(x: np.ndarray, pos: np.ndarray, base: float) -> np.ndarray:
    """Rotate rows x[t] (fp64, [T, d]) by the RoPE angle of position pos[t] (half-split pairs)."""
    d = x.shape[-1]
    half = d // 2
    theta = base ** (-2.0 * np.arange(half, dtype=np.float64) / d)
    ang = pos.astype(np.float64)[:, None] * theta[None, :]
    c, s = np.cos(ang), np.sin(ang)
    x1, x2 = x[:, :half], x[:, half:]
    return np.concatenate([x1 * c - x2 * s, x1 * s + x2 * c], axis=1)


def topic_sequence(w: Workload, b: int) -> np.ndarray:
    """z_t for t in [0, L0 + steps): piecewise-constant topics, Geometric piece lengths."""
    n = w.capacity
    rng = _rng(w, b, 0, 0, _TOPIC)
    z = np.empty(n, dtype=np.int32)
    t = 0
    while t < n:
        # draw in blocks to keep the Python loop short
        lens = rng.geometric(1.0 / w.topic_mean, size=4096)
        tops = rng.integers(0, N_TOPICS, size=4096)
        for ln, tp in zip(lens, tops):
            if t >= n:
                break
            z[t:t + ln] = tp
            t += ln
    return z


def topic_centres(w: Workload, layer: int, kvh: int) -> np.ndarray:
    return _rng(w, 0, layer, kvh, _CENTRES).standard_normal((N_TOPICS, w.head_dim))


@dataclass
class LayerInputs:
    """bf16 bit patterns (uint16) for one layer.

    k, v: [B, Hkv, L0 + steps, d] -- rows [0, L0) are the prefilled context, row L0 + s
          is the token appended at decode step s.
    q:    [steps, B, Hq, d] -- the query of decode step s sits at position L0 + s.
    """
    workload: Workload
    layer: int
    k: np.ndarray
    v: np.ndarray
    q: np.ndarray


_CHUNK = 16384  # rows per generation chunk (fixed: the drawn stream depends on it)


def _kv_head(w: Workload, z: np.ndarray, b: int, layer: int, g: int, rows: int,
             k_out: np.ndarray, v_out: np.ndarray) -> None:
    mu = topic_centres(w, layer, g)
    rk = _rng(w, b, layer, g, _KEYNOISE)
    rv = _rng(w, b, layer, g, _VALUES)
    for lo in range(0, rows, _CHUNK):
        hi = min(rows, lo + _CHUNK)
        eps = rk.standard_normal((hi - lo, w.head_dim), dtype=np.float32)
        x = mu[z[lo:hi]] + 0.5 * eps.astype(np.float64)
        k_out[lo:hi] = f32_to_bf16_bits(_rope(x, np.arange(lo, hi), w.rope_base).astype(np.float32))
        v_out[lo:hi] = f32_to_bf16_bits(rv.standard_normal((hi - lo, w.head_dim), dtype=np.float32))


def _queries(w: Workload, z: np.ndarray, b: int, layer: int) -> np.ndarray:
    """Queries [steps, Hq, d] (bf16 bits) of batch element b."""
    G, d = w.group, w.head_dim
    out = np.empty((w.steps, w.n_q_heads, d), dtype=np.uint16)
    pos = w.context + np.arange(w.steps)
    lo, hi = w.n_sink, w.context - w.n_recent  # indexed positions
    if hi <= lo:
        lo, hi = 0, w.context
    for g in range(w.n_kv_heads):
        mu = topic_centres(w, layer, g)
        tstar = _rng(w, b, layer, g, _QTARGET).integers(lo, hi, size=w.steps)
        for hh in range(G):
            h = g * G + hh
            xi = _rng(w, b, layer, h, _QNOISE).standard_normal((w.steps, d))
            delta = np.sqrt(0.5) * _rng(w, 0, layer, h, _QSHIFT).standard_normal(d)
            x = 0.8 * mu[z[tstar]] + xi + delta[None, :]
            out[:, h, :] = f32_to_bf16_bits(_rope(x, pos, w.rope_base).astype(np.float32))
    return out


def generate_layer(w: Workload, layer: int = 0, threads: int | None = None,
                   rows: int | None = None) -> LayerInputs:
    """Generate one layer's K, V (prefill + appended decode tokens) and decode queries.

    `rows` limits the generated K/V rows (default: L0 + steps); the queries always cover
    `steps` decode steps.
    """
    rows = w.capacity if rows is None else rows
    threads = threads or min(16, os.cpu_count() or 1)
    B, H, d = w.batch, w.n_kv_heads, w.head_dim
    k = np.empty((B, H, rows, d), dtype=np.uint16)
    v = np.empty((B, H, rows, d), dtype=np.uint16)
    q = np.empty((w.steps, B, w.n_q_heads, d), dtype=np.uint16)
    zs = [topic_sequence(w, b) for b in range(B)]

    def work(bg):
        b, g = bg
        _kv_head(w, zs[b], b, layer, g, rows, k[b, g], v[b, g])

    with ThreadPoolExecutor(max_workers=threads) as ex:
        list(ex.map(work, [(b, g) for b in range(B) for g in range(H)]))
    for b in range(B):
        q[:, b] = _queries(w, zs[b], b, layer)
    return LayerInputs(w, layer, k, v, q)


def training_queries(w: Workload, n_pos: int, layer: int = 0) -> np.ndarray:
    """Training queries [B, Hkv, n_pos * G, d] (bf16 bits): for each KV head, the queries of
    its G heads at the last n_pos prefill positions (t = i * G + hh for position
    L0 - n_pos + i and head g * G + hh)."""
    B, H, G, d = w.batch, w.n_kv_heads, w.group, w.head_dim
    out = np.empty((B, H, n_pos * G, d), dtype=np.uint16)
    pos = w.context - n_pos + np.arange(n_pos)
    lo, hi = w.n_sink, w.context - w.n_recent
    if hi <= lo:
        lo, hi = 0, w.context
    for b in range(B):
        z = topic_sequence(w, b)
        for g in range(H):
            mu = topic_centres(w, layer, g)
            tstar = _rng(w, b, layer, g, _TTARGET).integers(lo, hi, size=n_pos)
            for hh in range(G):
                h = g * G + hh
                xi = _rng(w, b, layer, h, _TNOISE).standard_normal((n_pos, d))
                delta = np.sqrt(0.5) * _rng(w, 0, layer, h, _QSHIFT).standard_normal(d)
                x = 0.8 * mu[z[tstar]] + xi + delta[None, :]
                out[b, g, hh::G] = f32_to_bf16_bits(_rope(x, pos, w.rope_base).astype(np.float32))
    return out
