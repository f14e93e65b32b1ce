"""Seeded synthetic inputs for latent-KV decode attention.

This module only draws numbers: per-head key ranks, the constant up-projection factors, latent
cache rows, dense K/V rows of exempt layers and decode queries. It holds no step of the method
(no RoPE, no attention, no rotation, no quantisation), so the HIP path and the oracle can both
consume its arrays without sharing any arithmetic of the method.

Shapes and value distributions follow the decode workloads of the STAR-KV pages: LLaMA-2-7B /
LongChat-7B layers (32 heads, head_dim 128, key ranks out of 128 per head, one joint value rank out
of 4096 per layer; Zhou, STAR-KV reading notes, section 4 / Fig. 2 and section 8.1), with the
latent column scale decaying like a singular-value spectrum (same notes, section 5.2 / Fig. 3).

Recipe (everything derives from numpy's PCG64 through explicit SeedSequence spawn keys, so a
slice of a workload can be redrawn on its own and the draw does not depend on the thread count):

* layer draw, ``SeedSequence(layer_seed, spawn_key=(layer, 0))``: key ranks (one choice per
  head, in head order), then per head ``B_k[h] = N(0,1)[r_h, d] / sqrt(r_h)`` in head order,
  then ``B_v = N(0,1)[r_v, H*d] / sqrt(r_v)``.
* cache rows of sequence b, ``SeedSequence(cache_seed, spawn_key=(layer, 1, b))``:
  ``Z_k = N(0,1)[T, R_k] * colstd_k`` then ``Z_v = N(0,1)[T, r_v] * colstd_v``; a dense layer
  draws ``K = N(0,1)[T, H*d]`` then ``V = N(0,1)[T, H*d]`` instead.
* queries, ``SeedSequence(cache_seed, spawn_key=(layer, 2))``: ``q = N(0,1)[B, H, d]`` (fp32).

``colstd`` is ``(j+1)**-power`` for column j counted inside each latent (each head's key latent
and the joint value latent), or 1 for i.i.d. draws. Values are drawn in fp32 and rounded once
(round-to-nearest-even) to the storage type.
"""
from __future__ import annotations

import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, field

import numpy as np

__all__ = [
    "Workload", "LayerDraw", "WORKLOADS", "to_bf16_bits", "bf16_bits_to_f32", "storage_numpy_dtype",
    "draw_layer", "draw_latent_cache", "draw_dense_cache", "draw_queries", "model_layers",
    "ModelLayer",
]


def to_bf16_bits(x32: np.ndarray) -> np.ndarray:
    """fp32 -> bfloat16 bit patterns, round-to-nearest-even (finite inputs)."""
    u = np.ascontiguousarray(x32, dtype=np.float32).view(np.uint32)
    bias = ((u >> np.uint32(16)) & np.uint32(1)) + np.uint32(0x7FFF)
    return ((u + bias) >> np.uint32(16)).astype(np.uint16)


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def storage_numpy_dtype(dtype: str):
    return {"f32": np.float32, "f16": np.float16, "bf16": np.uint16}[dtype]


def _store(x32: np.ndarray, dtype: str) -> np.ndarray:
    if dtype == "f32":
        return x32.astype(np.float32, copy=False)
    if dtype == "f16":
        return x32.astype(np.float16)
    if dtype == "bf16":
        return to_bf16_bits(x32)
    raise ValueError(f"unknown storage dtype {dtype!r}")


@dataclass(frozen=True)
class Workload:
    """One decode-attention workload: a layer (ranks, factors) plus a cache and queries."""
    name: str
    batch: int
    heads: int
    head_dim: int
    seq_len: int
    dtype: str                       # storage type of latents and factors: f32 | f16 | bf16
    layer_seed: int
    cache_seed: int
    value_rank: int
    key_rank_choices: tuple = ()     # per-head ranks drawn uniformly from this set ...
    fixed_key_rank: int = 0          # ... or all heads use this rank
    power: float = 0.0               # column std exponent (0 -> i.i.d.)
    quantized: bool = False          # cache stored as mixed 4/3-bit codes after rotation
    q_top_fraction: float = 0.25     # quantised caches: leading channels stored at 4 bits
    rope_base: float = 10000.0
    description: str = ""


# The five workloads. Names carry their sizes; the layer of the three LongChat-shaped workloads
# is the same draw (layer seed 1), only the cache differs.
WORKLOADS = {
    "tiny_b1_h4_d64_t256_f32": Workload(
        "tiny_b1_h4_d64_t256_f32", batch=1, heads=4, head_dim=64, seq_len=256, dtype="f32",
        layer_seed=0, cache_seed=0, value_rank=64, fixed_key_rank=16, power=0.0,
        description="tiny CPU-checkable decode, i.i.d. N(0,1), factors / sqrt(rank)"),
    "longchat_b16_t4096_f16": Workload(
        "longchat_b16_t4096_f16", batch=16, heads=32, head_dim=128, seq_len=4096, dtype="f16",
        layer_seed=1, cache_seed=1, value_rank=1024, key_rank_choices=(16, 32, 48, 64), power=0.5,
        description="LongChat-7B-shaped layer, key ranks U{16,32,48,64}, r_v 1024, power-law 0.5"),
    "longchat_b16_t32768_f16": Workload(
        "longchat_b16_t32768_f16", batch=16, heads=32, head_dim=128, seq_len=32768, dtype="f16",
        layer_seed=1, cache_seed=2, value_rank=1024, key_rank_choices=(16, 32, 48, 64), power=0.5,
        description="long-context decode, same layer, T=32768"),
    "longchat_b16_t16384_q43": Workload(
        "longchat_b16_t16384_q43", batch=16, heads=32, head_dim=128, seq_len=16384, dtype="f16",
        layer_seed=1, cache_seed=3, value_rank=1024, key_rank_choices=(16, 32, 48, 64), power=0.5,
        quantized=True,
        description="same layer, T=16384, latents rotated + mixed 4/3-bit (top 25% at 4 bits)"),
    # the same layer at the context lengths where the pages compare cache formats (8K, 16K):
    # binary16 latents, the mixed 4/3-bit cache and a uniform 4-bit cache (top fraction 1)
    "longchat_b16_t8192_f16": Workload(
        "longchat_b16_t8192_f16", batch=16, heads=32, head_dim=128, seq_len=8192, dtype="f16",
        layer_seed=1, cache_seed=5, value_rank=1024, key_rank_choices=(16, 32, 48, 64), power=0.5,
        description="same layer, T=8192, binary16 latents"),
    "longchat_b16_t16384_f16": Workload(
        "longchat_b16_t16384_f16", batch=16, heads=32, head_dim=128, seq_len=16384, dtype="f16",
        layer_seed=1, cache_seed=3, value_rank=1024, key_rank_choices=(16, 32, 48, 64), power=0.5,
        description="same layer and latents as the T=16384 quantised workload, binary16 latents"),
    "longchat_b16_t8192_q43": Workload(
        "longchat_b16_t8192_q43", batch=16, heads=32, head_dim=128, seq_len=8192, dtype="f16",
        layer_seed=1, cache_seed=5, value_rank=1024, key_rank_choices=(16, 32, 48, 64), power=0.5,
        quantized=True, description="same layer, T=8192, rotated, mixed 4/3-bit"),
    "longchat_b16_t8192_q4": Workload(
        "longchat_b16_t8192_q4", batch=16, heads=32, head_dim=128, seq_len=8192, dtype="f16",
        layer_seed=1, cache_seed=5, value_rank=1024, key_rank_choices=(16, 32, 48, 64), power=0.5,
        quantized=True, q_top_fraction=1.0, description="same layer, T=8192, rotated, uniform 4-bit"),
    "longchat_b16_t16384_q4": Workload(
        "longchat_b16_t16384_q4", batch=16, heads=32, head_dim=128, seq_len=16384, dtype="f16",
        layer_seed=1, cache_seed=3, value_rank=1024, key_rank_choices=(16, 32, 48, 64), power=0.5,
        quantized=True, q_top_fraction=1.0,
        description="same layer and latents as the T=16384 quantised workload, uniform 4-bit"),
}

# The 32-layer model step: batch 32, T 8192, layers 0, 1 and 31 dense fp16.
MODEL_STEP = dict(name="model32_b32_t8192_f16", seed=4, layers=32, dense_layers=(0, 1, 31),
                  batch=32, heads=32, head_dim=128, seq_len=8192,
                  key_rank_choices=(16, 32, 48, 64, 80, 96), value_rank_choices=(768, 1024, 1280),
                  power=0.5, dtype="f16")


@dataclass
class LayerDraw:
    key_ranks: np.ndarray            # int32 [H]
    bk: np.ndarray                   # [R_k, d] storage dtype
    bv: np.ndarray                   # [r_v, H*d] storage dtype
    value_rank: int
    dtype: str


def _colstd(ranks, power: float) -> np.ndarray:
    cols = np.concatenate([np.arange(r, dtype=np.float64) for r in ranks])
    if power == 0.0:
        return np.ones(cols.shape, np.float32)
    return ((cols + 1.0) ** (-power)).astype(np.float32)


def _layer_rng(seed: int, layer: int):
    return np.random.default_rng(np.random.SeedSequence(seed, spawn_key=(layer, 0)))


def draw_layer(w: Workload, layer: int = 0, key_ranks=None, value_rank=None) -> LayerDraw:
    rng = _layer_rng(w.layer_seed, layer)
    H, d = w.heads, w.head_dim
    if key_ranks is None:
        if w.key_rank_choices:
            key_ranks = rng.choice(np.asarray(w.key_rank_choices), size=H)
        else:
            key_ranks = np.full(H, w.fixed_key_rank)
    key_ranks = np.asarray(key_ranks, dtype=np.int32)
    r_v = int(value_rank if value_rank is not None else w.value_rank)
    bk = np.concatenate([rng.standard_normal((int(r), d), dtype=np.float32) / np.float32(np.sqrt(r))
                         for r in key_ranks])
    bv = rng.standard_normal((r_v, H * d), dtype=np.float32) / np.float32(np.sqrt(r_v))
    return LayerDraw(key_ranks, _store(bk, w.dtype), _store(bv, w.dtype), r_v, w.dtype)


def _workers() -> int:
    return max(1, min(16, os.cpu_count() or 1))


def _draw_rows(rng, T: int, colstd: np.ndarray, dtype: str, out: np.ndarray, chunk: int = 2048):
    C = colstd.shape[0]
    for t0 in range(0, T, chunk):
        t1 = min(T, t0 + chunk)
        x = rng.standard_normal((t1 - t0, C), dtype=np.float32)
        if not np.all(colstd == 1.0):
            x *= colstd
        out[t0:t1] = _store(x, dtype)


def draw_latent_cache(w: Workload, layer_draw: LayerDraw, layer: int = 0, batches=None,
                      seq_len: int | None = None):
    """Latent cache rows for the given sequences: zk [nb, T, R_k], zv [nb, T, r_v] (storage dtype).

    ``batches`` selects sequence indices (default all); each is drawn from its own stream, so a
    subset equals the corresponding slice of the full draw.
    """
    T = int(seq_len if seq_len is not None else w.seq_len)
    batches = list(range(w.batch)) if batches is None else list(batches)
    ranks = layer_draw.key_ranks
    ck = _colstd(ranks, w.power)
    cv = _colstd([layer_draw.value_rank], w.power)
    dt = storage_numpy_dtype(w.dtype)
    zk = np.empty((len(batches), T, ck.shape[0]), dt)
    zv = np.empty((len(batches), T, cv.shape[0]), dt)

    def one(i_b):
        i, b = i_b
        rng = np.random.default_rng(np.random.SeedSequence(w.cache_seed, spawn_key=(layer, 1, b)))
        _draw_rows(rng, T, ck, w.dtype, zk[i])
        _draw_rows(rng, T, cv, w.dtype, zv[i])

    with ThreadPoolExecutor(_workers()) as ex:
        list(ex.map(one, enumerate(batches)))
    return zk, zv


def draw_dense_cache(seed: int, layer: int, batch: int, seq_len: int, width: int, dtype="f16",
                     batches=None):
    """Dense exempt-layer rows: k, v [nb, T, H*d] i.i.d. N(0,1) (keys are pre-RoPE)."""
    batches = list(range(batch)) if batches is None else list(batches)
    dt = storage_numpy_dtype(dtype)
    k = np.empty((len(batches), seq_len, width), dt)
    v = np.empty((len(batches), seq_len, width), dt)
    ones = np.ones(width, np.float32)

    def one(i_b):
        i, b = i_b
        rng = np.random.default_rng(np.random.SeedSequence(seed, spawn_key=(layer, 1, b)))
        _draw_rows(rng, seq_len, ones, dtype, k[i])
        _draw_rows(rng, seq_len, ones, dtype, v[i])

    with ThreadPoolExecutor(_workers()) as ex:
        list(ex.map(one, enumerate(batches)))
    return k, v


def draw_queries(seed: int, layer: int, batch: int, heads: int, head_dim: int) -> np.ndarray:
    rng = np.random.default_rng(np.random.SeedSequence(seed, spawn_key=(layer, 2)))
    return rng.standard_normal((batch, heads, head_dim), dtype=np.float32)


@dataclass
class ModelLayer:
    index: int
    dense: bool
    workload: Workload                # shapes/seeds of this layer (seq_len = full T)
    key_ranks: np.ndarray = field(default=None)
    value_rank: int = 0


def model_layers(spec: dict | None = None):
    """Per-layer descriptors of the 32-layer decode step (ranks drawn per layer)."""
    s = dict(MODEL_STEP if spec is None else spec)
    out = []
    for l in range(s["layers"]):
        dense = l in s["dense_layers"]
        w = Workload(f"{s['name']}_layer{l}", batch=s["batch"], heads=s["heads"],
                     head_dim=s["head_dim"], seq_len=s["seq_len"], dtype=s["dtype"],
                     layer_seed=s["seed"], cache_seed=s["seed"], value_rank=0,
                     key_rank_choices=tuple(s["key_rank_choices"]), power=s["power"])
        if dense:
            out.append(ModelLayer(l, True, w))
            continue
        rng = _layer_rng(s["seed"], l)
        ranks = rng.choice(np.asarray(s["key_rank_choices"]), size=s["heads"]).astype(np.int32)
        r_v = int(rng.choice(np.asarray(s["value_rank_choices"])))
        out.append(ModelLayer(l, False, w, ranks, r_v))
    return out


def draw_model_layer(ml: ModelLayer) -> LayerDraw:
    """Factors of a latent model layer; ranks come from ``model_layers`` (same stream, after them)."""
    w = ml.workload
    rng = _layer_rng(w.layer_seed, ml.index)
    rng.choice(np.asarray(w.key_rank_choices), size=w.heads)         # ranks (already drawn)
    rng.choice(np.asarray(MODEL_STEP["value_rank_choices"]))          # value rank (already drawn)
    H, d = w.heads, w.head_dim
    bk = np.concatenate([rng.standard_normal((int(r), d), dtype=np.float32) / np.float32(np.sqrt(r))
                         for r in ml.key_ranks])
    bv = rng.standard_normal((ml.value_rank, H * d), dtype=np.float32) / np.float32(np.sqrt(ml.value_rank))
    return LayerDraw(ml.key_ranks, _store(bk, w.dtype), _store(bv, w.dtype), ml.value_rank, w.dtype)
