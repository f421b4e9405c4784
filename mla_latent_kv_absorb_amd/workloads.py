"""Seeded synthetic workloads for MLA absorb attention and latent-KV expansion.

This module only draws random inputs and rounds them to the storage type; it
holds none of the attention or expansion arithmetic.  Both the CPU oracle
(through the tests) and the HIP path consume exactly the arrays built here.

Shapes follow the DeepSeek-V3 MLA layout described on the page "Naive vs Absorb
Attention Implementations in DeepSeek-V3" (section "Memory Layout and Cache
Structure": kv_cache [batch, seq_len, kv_lora_rank], pe_cache [batch, seq_len,
qk_rope_head_dim]) and the kernelindex page "Latent KV expansion with split"
(128 heads, kv_lora_rank 512, expanded width 128 * (128 + 128)).

Recipe
------
* ``numpy.random.default_rng(seed)``; every tensor is drawn with
  ``standard_normal(dtype=float32)`` and scaled by the standard deviation.
  ``N(0, v)`` means variance ``v``.
* Attention workloads draw, in order: q_nope, q_pe, kv_cache, pe_cache, wkv_b.
* Expansion workloads draw, in order: c_kv, rms_w, wkv_b.
* Ragged batches take an attention workload (whose end_pos is the bound of the
  lengths) and draw the per-sequence lengths from their own generator:
  ``default_rng(seed).integers(lo, hi + 1, size=batch)``.
* bf16 workloads round each fp32 draw to bfloat16 with round-to-nearest-even;
  the arrays are returned as float32 holding exactly-representable bf16 values,
  so an upcast on either side is exact.
"""
from __future__ import annotations

import dataclasses
import math
from typing import Dict, Optional

import numpy as np

__all__ = [
    "AttnConfig",
    "ExpandConfig",
    "ATTN_CONFIGS",
    "EXPAND_CONFIGS",
    "round_to_bf16",
    "bf16_bits",
    "make_attn_inputs",
    "make_expand_inputs",
    "RAGGED_CONFIGS",
    "SKEWED_CONFIGS",
    "RAGGED_WORKLOADS",
    "ragged_lengths",
    "ragged_workload",
]


def bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bfloat16 (round-to-nearest-even); return the uint16 bit patterns."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    bias = ((u >> np.uint64(16)) & np.uint64(1)) + np.uint64(0x7FFF)
    return ((u + bias) >> np.uint64(16)).astype(np.uint16)


def round_to_bf16(x: np.ndarray) -> np.ndarray:
    """float32 -> nearest-even bfloat16 value, returned as float32."""
    bits = bf16_bits(x).astype(np.uint32) << np.uint32(16)
    return bits.view(np.float32)


@dataclasses.dataclass(frozen=True)
class AttnConfig:
    """One absorb-attention workload (decode when ``seqlen_q == 1``)."""

    name: str
    dtype: str  # "f32" or "bf16"
    batch: int
    seqlen_q: int
    n_heads: int
    kv_lora_rank: int
    qk_rope_head_dim: int
    qk_nope_head_dim: int
    v_head_dim: int
    end_pos: int
    cache_len: int  # allocated cache capacity (Tmax)
    cache_batch: int  # allocated cache rows (Bmax)
    wkv_b_var: float
    seed: int

    @property
    def softmax_scale(self) -> float:
        return 1.0 / math.sqrt(self.qk_nope_head_dim + self.qk_rope_head_dim)

    @property
    def start_pos(self) -> int:
        return self.end_pos - self.seqlen_q

    def replace(self, **kw) -> "AttnConfig":
        return dataclasses.replace(self, **kw)


@dataclasses.dataclass(frozen=True)
class ExpandConfig:
    """One latent-KV expansion workload."""

    name: str
    dtype: str
    n_tokens: int
    n_heads: int
    kv_lora_rank: int
    qk_nope_head_dim: int
    v_head_dim: int
    eps: float
    wkv_b_var: float
    rms_w_var: float
    seed: int

    def replace(self, **kw) -> "ExpandConfig":
        return dataclasses.replace(self, **kw)


_DSV3 = dict(n_heads=128, kv_lora_rank=512, qk_rope_head_dim=64, qk_nope_head_dim=128, v_head_dim=128)

ATTN_CONFIGS: Dict[str, AttnConfig] = {
    # Tiny fp32 decode: batch 1, 4 heads, latent 64, rope 16, nope 32, v 32, 128 cached tokens.
    "tiny_f32": AttnConfig(
        "tiny_f32", "f32", batch=1, seqlen_q=1, n_heads=4, kv_lora_rank=64, qk_rope_head_dim=16,
        qk_nope_head_dim=32, v_head_dim=32, end_pos=128, cache_len=128, cache_batch=1,
        wkv_b_var=1.0 / 64, seed=0),
    # DeepSeek-V3 decode shape: 32 sequences x 4096 cached tokens, 128 heads.
    "dsv3_decode": AttnConfig(
        "dsv3_decode", "bf16", batch=32, seqlen_q=1, end_pos=4096, cache_len=4096, cache_batch=32,
        wkv_b_var=1.0 / 512, seed=1, **_DSV3),
    # Long context decode: 4 sequences x 32768 cached tokens.
    "long_decode": AttnConfig(
        "long_decode", "bf16", batch=4, seqlen_q=1, end_pos=32768, cache_len=32768, cache_batch=4,
        wkv_b_var=1.0 / 512, seed=2, **_DSV3),
    # Chunked prefill: 2 sequences, 512 new tokens at start_pos 3584, causal within the chunk.
    "chunk_prefill": AttnConfig(
        "chunk_prefill", "bf16", batch=2, seqlen_q=512, end_pos=4096, cache_len=4096, cache_batch=2,
        wkv_b_var=1.0 / 512, seed=3, **_DSV3),
}

EXPAND_CONFIGS: Dict[str, ExpandConfig] = {
    # Small fp32 expansion drawn together with the tiny attention workload's shapes.
    "tiny_f32": ExpandConfig(
        "tiny_f32", "f32", n_tokens=128, n_heads=4, kv_lora_rank=64, qk_nope_head_dim=32,
        v_head_dim=32, eps=1e-6, wkv_b_var=1.0 / 64, rms_w_var=0.02, seed=0),
    # DeepSeek-V3 latent KV expansion: 8192 tokens, 512 -> 128 * (128 + 128).
    "dsv3_expand": ExpandConfig(
        "dsv3_expand", "bf16", n_tokens=8192, n_heads=128, kv_lora_rank=512, qk_nope_head_dim=128,
        v_head_dim=128, eps=1e-6, wkv_b_var=1.0 / 512, rms_w_var=0.02, seed=4),
}


# Ragged-batch workloads: (attention workload, lowest length, highest length, seed of the lengths).
# The decode one stands in for a serving batch whose sequences have different context lengths.
RAGGED_CONFIGS: Dict[str, tuple] = {
    "ragged_decode": ("dsv3_decode", 256, 4096, 5),
}


# Skewed ragged workloads: (attention workload, sequences at the long length, long length, short
# length).  A few long contexts among many short ones: the batch in which one split count for
# every sequence leaves most workgroups idle.
SKEWED_CONFIGS: Dict[str, tuple] = {
    "skewed_decode": ("dsv3_decode", 4, 4096, 64),
}

RAGGED_WORKLOADS = list(RAGGED_CONFIGS) + list(SKEWED_CONFIGS)


def ragged_lengths(batch: int, lo: int, hi: int, seed: int) -> np.ndarray:
    """Per-sequence lengths drawn uniformly from [lo, hi] (int32)."""
    return np.random.default_rng(seed).integers(lo, hi + 1, size=batch).astype(np.int32)


def ragged_workload(name: str):
    """(attention workload name, int32 lengths [batch]) of a ragged or skewed workload."""
    if name in RAGGED_CONFIGS:
        base, lo, hi, seed = RAGGED_CONFIGS[name]
        return base, ragged_lengths(ATTN_CONFIGS[base].batch, lo, hi, seed)
    base, n_long, long_len, short_len = SKEWED_CONFIGS[name]
    batch = ATTN_CONFIGS[base].batch
    return base, np.array([long_len] * n_long + [short_len] * (batch - n_long), dtype=np.int32)


def _draw(rng: np.random.Generator, shape, std: float, mean: float = 0.0) -> np.ndarray:
    x = rng.standard_normal(shape, dtype=np.float32)
    if std != 1.0:
        x *= np.float32(std)
    if mean != 0.0:
        x += np.float32(mean)
    return x


def _store(x: np.ndarray, dtype: str) -> np.ndarray:
    if dtype == "f32":
        return x
    if dtype == "bf16":
        return round_to_bf16(x)
    raise ValueError(f"unknown dtype {dtype!r}")


def make_attn_inputs(cfg: AttnConfig, seed: Optional[int] = None) -> Dict[str, np.ndarray]:
    """Draw q_nope [B,S,H,Dn], q_pe [B,S,H,R], kv_cache [Bmax,Tmax,C], pe_cache [Bmax,Tmax,R],
    wkv_b [H*(Dn+Dv), C] as float32 arrays holding values of the workload's storage type."""
    rng = np.random.default_rng(cfg.seed if seed is None else seed)
    B, S, H = cfg.batch, cfg.seqlen_q, cfg.n_heads
    C, R, Dn, Dv = cfg.kv_lora_rank, cfg.qk_rope_head_dim, cfg.qk_nope_head_dim, cfg.v_head_dim
    out = {
        "q_nope": _draw(rng, (B, S, H, Dn), 1.0),
        "q_pe": _draw(rng, (B, S, H, R), 1.0),
        "kv_cache": _draw(rng, (cfg.cache_batch, cfg.cache_len, C), 1.0),
        "pe_cache": _draw(rng, (cfg.cache_batch, cfg.cache_len, R), 1.0),
        "wkv_b": _draw(rng, (H * (Dn + Dv), C), math.sqrt(cfg.wkv_b_var)),
    }
    return {k: _store(v, cfg.dtype) for k, v in out.items()}


def make_expand_inputs(cfg: ExpandConfig, seed: Optional[int] = None) -> Dict[str, np.ndarray]:
    """Draw c_kv [T,C], rms_w [C] (= 1 + N(0, rms_w_var)), wkv_b [H*(Dn+Dv), C]."""
    rng = np.random.default_rng(cfg.seed if seed is None else seed)
    C = cfg.kv_lora_rank
    out = {
        "c_kv": _draw(rng, (cfg.n_tokens, C), 1.0),
        "rms_w": _draw(rng, (C,), math.sqrt(cfg.rms_w_var), mean=1.0),
        "wkv_b": _draw(rng, (cfg.n_heads * (cfg.qk_nope_head_dim + cfg.v_head_dim), C),
                       math.sqrt(cfg.wkv_b_var)),
    }
    return {k: _store(v, cfg.dtype) for k, v in out.items()}
