"""Seeded synthetic inputs shared by the oracle tests, the GPU parity tests and the benchmark.

This module only draws random numbers and rounds them to the storage format; it contains none of
the attention arithmetic.  Both the HIP path and the CPU oracle consume exactly the bits produced
here (bf16 bit patterns, or fp32 values), so input rounding is common to both sides.

Workload recipes (token-major layout ``[B, S, H, D]``, as a sequence of tokens each carrying H heads):

* ``demo``: the four-device, 8-token-block, head-dim-16 demonstration on the Ultralytics glossary
  page "Ring Attention" (section "Como funciona a atenção em anel"): ``torch.manual_seed(0)`` then a
  single ``randn(3, 32, 16)`` draw split into q, k, v, fp32.
* ``noncausal_16k``: B=1, S=16384, 8 heads, D=128, P=8 shards of 2048, i.i.d. N(0,1), bf16.
* ``causal_32k``: B=1, S=32768, 32 heads, D=128, P=8 shards of 4096, N(0,1) scaled by 0.5, bf16.
* ``causal_striped_64k``: B=1, S=65536, 32 query heads, 8 KV heads, D=128, P=8, N(0,1), bf16.
* ``causal_1m_shard``: one device's share of a 1,048,576-token ring of 32 shards (n=32768):
  local queries = the last shard, K/V = the whole sequence, 8 heads, D=128, N(0,1), bf16;
  ``causal_1m_shard_host`` the same with the key/value source in pinned host memory.

Feed-forward workloads (the blockwise feed-forward after attention; the pages give no sizes, so
d_model = Hq * D of an attention workload and d_ff = 4 d_model): x ~ N(0, 1) (an attention output
has O(1) entries), w1 ~ N(0, 1/d_model), w2 ~ N(0, 1/d_ff) (variance-preserving initialisation, so
the hidden and output activations are O(1) too), b1, b2 ~ N(0, 0.1^2), all rounded to bf16.

* ``ffn_16k``: the 16384 tokens of ``noncausal_16k``'s output, d_model 1024, d_ff 4096.
* ``ffn_32h_4k``: 4096 tokens of the 32-head configurations, d_model 4096, d_ff 16384.
"""
from __future__ import annotations

import dataclasses

import numpy as np

__all__ = [
    "Workload", "WORKLOADS", "bf16_bits", "bf16_to_f32", "normal_bf16", "normal_f32",
    "demo_qkv", "workload_qkv", "workload_dout", "FfnWorkload", "FFN_WORKLOADS", "ffn_inputs",
]


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    B: int
    S: int          # full sequence length
    P: int          # ring size (number of shards)
    Hq: int
    Hkv: int
    D: int
    causal: bool
    layout: str     # "contiguous", "striped" or "zigzag"
    dtype: str      # "f32" or "bf16"
    seed: int
    sigma: float = 1.0
    # for the one-device share: which shard is local (None = all shards emulated on one GPU)
    local_shard: int | None = None
    # the backward ring (gradients for a seeded output gradient) instead of the forward
    backward: bool = False
    # key/value source in pinned host memory instead of HBM (every hop a host-to-device copy)
    kv_host: bool = False

    @property
    def n(self) -> int:
        return self.S // self.P

    def visible_pairs(self) -> int:
        """Number of (query, key) pairs that attend (per batch element and query head)."""
        if self.local_shard is None:
            return self.S * (self.S + 1) // 2 if self.causal else self.S * self.S
        n, i = self.n, self.local_shard
        if not self.causal:
            return n * self.S
        return i * n * n + n * (n + 1) // 2

    def flops(self) -> float:
        """Algorithmic FLOPs: 2*D for Q.K^T plus 2*D for P.V per visible pair; the backward counts
        five such products (Q.K^T again, dO.V^T, P^T.dO, dS^T.Q, dS.K), 10*D per visible pair."""
        return (10.0 if self.backward else 4.0) * self.D * self.Hq * self.B * self.visible_pairs()


WORKLOADS = {
    "demo": Workload("demo", 1, 32, 4, 1, 1, 16, False, "contiguous", "f32", 0),
    "noncausal_16k": Workload("noncausal_16k", 1, 16384, 8, 8, 8, 128, False, "contiguous", "bf16", 2000),
    "causal_32k": Workload("causal_32k", 1, 32768, 8, 32, 32, 128, True, "contiguous", "bf16", 3000, 0.5),
    "causal_striped_64k": Workload("causal_striped_64k", 1, 65536, 8, 32, 8, 128, True, "striped", "bf16", 4000),
    "causal_contig_64k": Workload("causal_contig_64k", 1, 65536, 8, 32, 8, 128, True, "contiguous", "bf16", 4000),
    "causal_zigzag_64k": Workload("causal_zigzag_64k", 1, 65536, 8, 32, 8, 128, True, "zigzag", "bf16", 4000),
    "causal_1m_shard": Workload("causal_1m_shard", 1, 1048576, 32, 8, 8, 128, True, "contiguous", "bf16", 5000,
                                local_shard=31),
    "causal_1m_shard_host": Workload("causal_1m_shard_host", 1, 1048576, 32, 8, 8, 128, True, "contiguous", "bf16",
                                     5000, local_shard=31, kv_host=True),
    "bwd_noncausal_16k": Workload("bwd_noncausal_16k", 1, 16384, 8, 8, 8, 128, False, "contiguous", "bf16", 2000,
                                  backward=True),
    "bwd_causal_striped_64k": Workload("bwd_causal_striped_64k", 1, 65536, 8, 32, 8, 128, True, "striped", "bf16",
                                       4000, backward=True),
    "bwd_causal_zigzag_64k": Workload("bwd_causal_zigzag_64k", 1, 65536, 8, 32, 8, 128, True, "zigzag", "bf16",
                                      4000, backward=True),
}


def bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bfloat16 (round to nearest, ties to even); return the uint16 bit patterns."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32).astype(np.uint64)
    rounding_bias = ((u >> 16) & 1) + 0x7FFF
    out = ((u + rounding_bias) >> 16).astype(np.uint16)
    nan = np.isnan(x)
    if nan.any():
        out[nan] = 0x7FC0
    return out


def bf16_to_f32(bits: np.ndarray) -> np.ndarray:
    """Exact widening of bfloat16 bit patterns to float32."""
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def normal_f32(seed: int, shape, sigma: float = 1.0, chunk: int = 1 << 24) -> np.ndarray:
    """i.i.d. N(0, sigma^2) float32 from numpy's PCG64 generator, drawn in chunks to bound memory."""
    rng = np.random.default_rng(seed)
    total = int(np.prod(shape))
    out = np.empty(total, dtype=np.float32)
    for s in range(0, total, chunk):
        e = min(total, s + chunk)
        out[s:e] = rng.standard_normal(e - s, dtype=np.float32)
        if sigma != 1.0:
            out[s:e] *= np.float32(sigma)
    return out.reshape(shape)


def normal_bf16(seed: int, shape, sigma: float = 1.0, chunk: int = 1 << 24) -> np.ndarray:
    """i.i.d. N(0, sigma^2) rounded to bfloat16; returns uint16 bit patterns."""
    rng = np.random.default_rng(seed)
    total = int(np.prod(shape))
    out = np.empty(total, dtype=np.uint16)
    for s in range(0, total, chunk):
        e = min(total, s + chunk)
        x = rng.standard_normal(e - s, dtype=np.float32)
        if sigma != 1.0:
            x *= np.float32(sigma)
        out[s:e] = bf16_bits(x)
    return out.reshape(shape)


def demo_qkv():
    """The demonstration's inputs: seed 0, one randn(3, 32, 16) draw (torch CPU generator), fp32.

    Returns q, k, v as float32 numpy arrays of shape [32, 16].
    """
    import torch
    g = torch.Generator().manual_seed(0)
    qkv = torch.randn(3, 32, 16, generator=g)
    return qkv[0].numpy().copy(), qkv[1].numpy().copy(), qkv[2].numpy().copy()


def workload_qkv(w: Workload):
    """Seeded inputs for workload ``w`` in token order ``[B, S, H, D]``.

    bf16 workloads return uint16 bit patterns; f32 workloads return float32.  Seeds are
    ``w.seed + 0/1/2`` for q/k/v.  For the one-device share, q covers only the local shard's
    tokens while k/v cover the whole sequence.
    """
    if w.name == "demo":
        q, k, v = demo_qkv()
        return q.reshape(1, 32, 1, 16), k.reshape(1, 32, 1, 16), v.reshape(1, 32, 1, 16)
    gen = normal_bf16 if w.dtype == "bf16" else normal_f32
    sq = w.n if w.local_shard is not None else w.S
    q = gen(w.seed + 0, (w.B, sq, w.Hq, w.D), w.sigma)
    k = gen(w.seed + 1, (w.B, w.S, w.Hkv, w.D), w.sigma)
    v = gen(w.seed + 2, (w.B, w.S, w.Hkv, w.D), w.sigma)
    return q, k, v


def workload_dout(w: Workload):
    """Seeded output gradient dO for a backward workload, token order [B, S, Hq, D] (seed ``w.seed + 3``)."""
    gen = normal_bf16 if w.dtype == "bf16" else normal_f32
    sq = w.n if w.local_shard is not None else w.S
    return gen(w.seed + 3, (w.B, sq, w.Hq, w.D), w.sigma)


@dataclasses.dataclass(frozen=True)
class FfnWorkload:
    name: str
    tokens: int
    d_model: int
    d_ff: int
    block_tokens: int
    activation: str  # "gelu" or "relu"
    seed: int

    def flops(self) -> float:
        """Algorithmic FLOPs of the two projections: 2 * d_model * d_ff per token each."""
        return 4.0 * self.tokens * self.d_model * self.d_ff


FFN_WORKLOADS = {
    "ffn_16k": FfnWorkload("ffn_16k", 16384, 1024, 4096, 16384, "gelu", 6000),
    "ffn_32h_4k": FfnWorkload("ffn_32h_4k", 4096, 4096, 16384, 4096, "gelu", 6100),
}


def ffn_inputs(seed: int, tokens: int, d_model: int, d_ff: int):
    """x [tokens, d_model], w1 [d_ff, d_model], b1 [d_ff], w2 [d_model, d_ff], b2 [d_model] as bf16 bit
    patterns (seeds seed + 0..4; weights in nn.Linear layout, one row per output feature)."""
    x = normal_bf16(seed, (tokens, d_model))
    w1 = normal_bf16(seed + 1, (d_ff, d_model), 1.0 / np.sqrt(d_model))
    b1 = normal_bf16(seed + 2, (d_ff,), 0.1)
    w2 = normal_bf16(seed + 3, (d_model, d_ff), 1.0 / np.sqrt(d_ff))
    b2 = normal_bf16(seed + 4, (d_model,), 0.1)
    return x, w1, b1, w2, b2
