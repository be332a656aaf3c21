"""Seeded synthetic inputs for the fused GQA attention workloads.

This module only draws numbers and lays them out in the shapes the attention
calls take. It holds none of the attention arithmetic, so both the fp64 oracle
(``oracle/``) and the HIP library (``attention_gqa_online_amd``) can be fed
from it without sharing any code with each other.

Recipe (same for every workload): ``numpy.random.default_rng(seed)`` (PCG64)
draws ``standard_normal(shape, dtype=float32)`` arrays, multiplied by the
float32 value of ``sigma`` (a standard deviation), in the order Q (or q), K, V.
The spiky decode workload then picks ``floor(spike_frac * B * Hkv * max_seq)``
distinct ``(b, g, s)`` rows of the K cache over *all* positions, in and out of
the sliding window, and multiplies those K rows by ``spike_scale``.

Layouts:
  prefill  Q ``[m, q_stride]``, K and V ``[m, kv_stride]`` (row-major; the
           columns past ``num_q_heads*head_dim`` / ``kv_heads*head_dim`` are
           filled too, as they would be inside a fused projection output).
  decode   q ``[batch, num_heads, head_dim]``,
           K and V caches ``[batch, kv_heads, max_seq, head_dim]``.
  append   K and V sources ``[batch, kv_heads, head_dim]``.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field, replace

import numpy as np

__all__ = [
    "PrefillWorkload",
    "DecodeWorkload",
    "WORKLOADS",
    "prefill_inputs",
    "decode_inputs",
    "append_inputs",
    "normal",
]


@dataclass(frozen=True)
class PrefillWorkload:
    """Shape of one causal prefill call (packed, strided rows)."""

    name: str
    m: int
    num_q_heads: int
    heads_per_kv: int
    head_dim: int
    q_stride: int
    kv_stride: int
    sigma: float = 1.0
    seed: int = 0

    @property
    def kv_heads(self) -> int:
        return self.num_q_heads // self.heads_per_kv

    def flops(self) -> int:
        """Algorithmic FLOPs: 2*d per score and 2*d per weighted V row, over
        the m(m+1)/2 causal (query, key) pairs of every Q head."""
        return 2 * self.head_dim * self.m * (self.m + 1) * self.num_q_heads

    def with_(self, **kw) -> "PrefillWorkload":
        return replace(self, **kw)


@dataclass(frozen=True)
class DecodeWorkload:
    """Shape of one single-query decode call over a batch of KV caches."""

    name: str
    batch: int
    num_heads: int
    kv_heads: int
    head_dim: int
    max_seq: int
    total_seq: int
    window: int = 0
    sigma: float = 1.0
    spike_frac: float = 0.0
    spike_scale: float = 1.0
    seed: int = 0
    scale: float = field(default=float("nan"))

    def __post_init__(self):
        if math.isnan(self.scale):
            # the decode configs state scale = 1/sqrt(head_dim), as a float32
            s = np.float32(1.0) / np.sqrt(np.float32(self.head_dim))
            object.__setattr__(self, "scale", float(s))

    @property
    def heads_per_kv(self) -> int:
        return self.num_heads // self.kv_heads

    @property
    def window_start(self) -> int:
        if self.window > 0 and self.total_seq > self.window:
            return self.total_seq - self.window
        return 0

    @property
    def attended(self) -> int:
        return self.total_seq - self.window_start

    def kv_bytes(self) -> int:
        """Algorithmic HBM bytes: each attended K and V row of every
        (sequence, KV head) read once, fp32."""
        return 2 * self.batch * self.kv_heads * self.attended * self.head_dim * 4

    def flops(self) -> int:
        return 4 * self.head_dim * self.attended * self.num_heads * self.batch

    def with_(self, **kw) -> "DecodeWorkload":
        return replace(self, **kw)


# The five synthetic workloads of the benchmark, named by what they are.
WORKLOADS = {
    "prefill_hq4_hkv2_d32_m16": PrefillWorkload(
        "prefill_hq4_hkv2_d32_m16", m=16, num_q_heads=4, heads_per_kv=2,
        head_dim=32, q_stride=128, kv_stride=64, sigma=1.0, seed=1001),
    "decode_b32_hq12_hkv2_d128_t4096": DecodeWorkload(
        "decode_b32_hq12_hkv2_d128_t4096", batch=32, num_heads=12, kv_heads=2,
        head_dim=128, max_seq=4096, total_seq=4096, window=0, sigma=1.0,
        seed=1002),
    "prefill_hq28_hkv4_d128_m2048": PrefillWorkload(
        "prefill_hq28_hkv4_d128_m2048", m=2048, num_q_heads=28, heads_per_kv=7,
        head_dim=128, q_stride=3584, kv_stride=512, sigma=1.0, seed=1003),
    "decode_b16_hq32_hkv8_d128_t32768_w4096": DecodeWorkload(
        "decode_b16_hq32_hkv8_d128_t32768_w4096", batch=16, num_heads=32,
        kv_heads=8, head_dim=128, max_seq=32768, total_seq=32768, window=4096,
        sigma=0.5, spike_frac=0.01, spike_scale=8.0, seed=1004),
    "prefill_hq64_hkv8_d128_m16384": PrefillWorkload(
        "prefill_hq64_hkv8_d128_m16384", m=16384, num_q_heads=64,
        heads_per_kv=8, head_dim=128, q_stride=8192, kv_stride=1024,
        sigma=1.0, seed=1005),
}


def normal(rng: np.random.Generator, shape, sigma: float) -> np.ndarray:
    """float32 N(0, sigma^2) draws (sigma is a standard deviation)."""
    a = rng.standard_normal(shape, dtype=np.float32)
    if sigma != 1.0:
        a *= np.float32(sigma)
    return a


def prefill_inputs(w: PrefillWorkload, seed: int | None = None):
    """Q ``[m, q_stride]``, K ``[m, kv_stride]``, V ``[m, kv_stride]`` float32."""
    rng = np.random.default_rng(w.seed if seed is None else seed)
    q = normal(rng, (w.m, w.q_stride), w.sigma)
    k = normal(rng, (w.m, w.kv_stride), w.sigma)
    v = normal(rng, (w.m, w.kv_stride), w.sigma)
    return q, k, v


def decode_inputs(w: DecodeWorkload, seed: int | None = None):
    """q ``[B, Hq, d]``, K and V caches ``[B, Hkv, max_seq, d]`` float32.

    Rows past ``total_seq`` are filled too (a cache is allocated whole); the
    spike rows are drawn over every ``(b, g, s)`` row of the K cache.
    """
    rng = np.random.default_rng(w.seed if seed is None else seed)
    q = normal(rng, (w.batch, w.num_heads, w.head_dim), w.sigma)
    shape = (w.batch, w.kv_heads, w.max_seq, w.head_dim)
    k = normal(rng, shape, w.sigma)
    v = normal(rng, shape, w.sigma)
    if w.spike_frac > 0.0:
        n_rows = w.batch * w.kv_heads * w.max_seq
        n_spike = int(math.floor(w.spike_frac * n_rows))
        rows = rng.choice(n_rows, size=n_spike, replace=False)
        k.reshape(n_rows, w.head_dim)[rows] *= np.float32(w.spike_scale)
    return q, k, v


def append_inputs(batch: int, kv_heads: int, head_dim: int, seed: int,
                  sigma: float = 1.0):
    """New K and V rows ``[B, Hkv, d]`` float32 for one cache append."""
    rng = np.random.default_rng(seed)
    k = normal(rng, (batch, kv_heads, head_dim), sigma)
    v = normal(rng, (batch, kv_heads, head_dim), sigma)
    return k, v


def seq_lengths(batch: int, max_len: int, seed: int, min_len: int = 1,
                idle: int = 0):
    """Per-sequence lengths ``[batch]`` uint32 for a mixed-length decode
    batch: uniform in [min_len, max_len], the longest forced to max_len
    (so the batch bound is reached), and ``idle`` slots of length 0."""
    rng = np.random.default_rng(seed)
    lens = rng.integers(min_len, max_len + 1, size=batch).astype(np.uint32)
    if batch:
        lens[int(rng.integers(batch))] = max_len
    if idle:
        free = np.flatnonzero(lens != max_len)
        lens[rng.choice(free, size=min(idle, free.size), replace=False)] = 0
    return lens


def rope_tables(head_dim: int, position: int, base: float = 10000.0):
    """cos/sin tables ``[head_dim/2]`` float32 for one position: pair i turns
    by position * base^(-2i/head_dim) (the usual geometric frequency
    schedule; the fused rotary decode takes the tables as given inputs)."""
    i = np.arange(head_dim // 2, dtype=np.float64)
    theta = position * base ** (-2.0 * i / head_dim)
    return np.cos(theta).astype(np.float32), np.sin(theta).astype(np.float32)


# ---------------------------------------------------------------------------
# On-device generation for timing runs (large caches in milliseconds). Same
# distributions and layouts as above, drawn with torch's seeded generator on
# the GPU; these arrays are for throughput measurement, the numpy ones above
# are what the oracle checks.

def _torch_normal(gen, shape, sigma, device):
    import torch
    a = torch.randn(shape, generator=gen, device=device, dtype=torch.float32)
    if sigma != 1.0:
        a.mul_(sigma)
    return a


def prefill_inputs_device(w: PrefillWorkload, seed: int, device):
    import torch
    gen = torch.Generator(device=device)
    gen.manual_seed(seed)
    q = _torch_normal(gen, (w.m, w.q_stride), w.sigma, device)
    k = _torch_normal(gen, (w.m, w.kv_stride), w.sigma, device)
    v = _torch_normal(gen, (w.m, w.kv_stride), w.sigma, device)
    return q, k, v


def decode_inputs_device(w: DecodeWorkload, seed: int, device):
    import torch
    gen = torch.Generator(device=device)
    gen.manual_seed(seed)
    q = _torch_normal(gen, (w.batch, w.num_heads, w.head_dim), w.sigma, device)
    shape = (w.batch, w.kv_heads, w.max_seq, w.head_dim)
    k = _torch_normal(gen, shape, w.sigma, device)
    v = _torch_normal(gen, shape, w.sigma, device)
    if w.spike_frac > 0.0:
        n_rows = w.batch * w.kv_heads * w.max_seq
        n_spike = int(math.floor(w.spike_frac * n_rows))
        rows = torch.randperm(n_rows, generator=gen, device=device)[:n_spike]
        k.view(n_rows, w.head_dim)[rows] *= w.spike_scale
    return q, k, v
