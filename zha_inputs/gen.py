"""Seeded input recipe for the five synthetic workloads.

Every draw comes from its own PCG64 stream addressed by a SeedSequence spawn
key, so one (sequence, KV head) block can be produced without drawing the
others.  The streams are:

  (0,)        reference queries  [Hkv][R][d]  ~ N(0, 1/d), kept in fp32
  (1,)        per-(b, g) key scale s ~ U[0.5, 2]   (1 where the workload has none)
  (2, b, g)   keys K ~ s * N(0, 1) [N][d], then values V ~ N(0, 1) [N][d]
  (3,)        decode queries [T][B][Hq][d] ~ N(0, 1) / sqrt(d)
  (4, b, g)   needles: (query step t, query head h in group g, position >= 1)
  (5, b, g)   rows appended during decode: K ~ s * N(0, 1), then V ~ N(0, 1)

Queries, keys and values are rounded to the workload's storage dtype (bf16,
round-to-nearest-even) before use; a needle key is s * 4 * q / |q| for the
stored (rounded) query it is planted for, then rounded itself.  Positions of
the needles are distinct and never 0, so the attention sink is never a needle.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field

import numpy as np


@dataclass(frozen=True)
class Config:
    name: str
    seed: int
    batch: int
    n_tokens: int            # keys/values per sequence before any decode-time append
    n_q_heads: int
    n_kv_heads: int
    head_dim: int
    chunk: int               # C: children per node (tokens per leaf chunk)
    levels: int              # L: summary levels; a top node covers C**L tokens
    n_refs: int              # R: reference queries per KV head
    p: tuple = (0.95,)       # routing mass fractions
    n_queries: int = 8       # decode queries (steps) T
    needles_per_unit: int = 0
    needles_per_query: int = 0
    dtype: str = "bf16"      # storage dtype of q, K, V and of the stored summaries m
    head_scale: bool = True
    append_steps: int = 0    # rows appended per sequence (one per decode step)
    parity_queries: int = 8  # decode steps checked against the oracle
    description: str = field(default="", compare=False)

    @property
    def group(self) -> int:
        return self.n_q_heads // self.n_kv_heads

    @property
    def max_tokens(self) -> int:
        return self.n_tokens + self.append_steps


CONFIGS = {
    "tiny_deep_f32": Config(
        name="tiny_deep_f32", seed=0, batch=1, n_tokens=4096, n_q_heads=1, n_kv_heads=1,
        head_dim=64, chunk=4, levels=3, n_refs=4, p=(0.95,), n_queries=8,
        needles_per_query=3, dtype="f32", head_scale=False,
        description="N=4096, 1 head, d=64, C=4 L=3 R=4 p=0.95, fp32"),
    "deep_256k": Config(
        name="deep_256k", seed=1, batch=1, n_tokens=262144, n_q_heads=32, n_kv_heads=4,
        head_dim=128, chunk=4, levels=6, n_refs=16, p=(0.95,), n_queries=64,
        needles_per_unit=32, dtype="bf16",
        description="N=262144, 32q/4kv heads, d=128, C=4 L=6 R=16 p=0.95, bf16"),
    "wide_256k": Config(
        name="wide_256k", seed=1, batch=1, n_tokens=262144, n_q_heads=32, n_kv_heads=4,
        head_dim=128, chunk=256, levels=1, n_refs=16, p=(0.95,), n_queries=64,
        needles_per_unit=32, dtype="bf16",
        description="N=262144, 32q/4kv heads, d=128, C=256 L=1 R=16 p=0.95, bf16"),
    "deep_1m": Config(
        name="deep_1m", seed=3, batch=1, n_tokens=1048576, n_q_heads=32, n_kv_heads=4,
        head_dim=128, chunk=4, levels=7, n_refs=16, p=(0.95,), n_queries=64,
        needles_per_unit=32, dtype="bf16",
        description="N=1048576, 32q/4kv heads, d=128, C=4 L=7 R=16 p=0.95, bf16"),
    "batch8_append_512k": Config(
        name="batch8_append_512k", seed=4, batch=8, n_tokens=524288, n_q_heads=32,
        n_kv_heads=4, head_dim=128, chunk=4, levels=6, n_refs=4, p=(0.7, 0.9, 0.99),
        n_queries=1024, needles_per_unit=32, dtype="bf16", append_steps=1024,
        description="8 x N=524288 growing by 1024, 32q/4kv heads, d=128, C=4 L=6 R=4, "
                    "p in {0.7, 0.9, 0.99}, bf16"),
}


def get_config(name: str, **overrides) -> Config:
    cfg = CONFIGS[name]
    if overrides:
        cfg = Config(**{**cfg.__dict__, **overrides})
    return cfg


# ----------------------------------------------------------------------------- rounding

def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """fp32 -> bf16 bit patterns, round to nearest even (finite inputs)."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    bias = ((u >> np.uint32(16)) & np.uint32(1)) + np.uint32(0x7FFF)
    return ((u + bias) >> np.uint32(16)).astype(np.uint16)


def bf16_to_f32(bits: np.ndarray) -> np.ndarray:
    return (np.ascontiguousarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def bf16_round(x: np.ndarray) -> np.ndarray:
    return bf16_to_f32(f32_to_bf16_bits(x))


def _store(cfg: Config, x: np.ndarray) -> np.ndarray:
    x = np.asarray(x, dtype=np.float32)
    return bf16_round(x) if cfg.dtype == "bf16" else np.ascontiguousarray(x)


# ----------------------------------------------------------------------------- streams

def _rng(cfg: Config, *key: int) -> np.random.Generator:
    ss = np.random.SeedSequence(cfg.seed, spawn_key=tuple(int(k) for k in key))
    return np.random.Generator(np.random.PCG64(ss))


def refs(cfg: Config) -> np.ndarray:
    """Reference queries [Hkv][R][d], fp32, entries ~ N(0, 1/d)."""
    r = _rng(cfg, 0).standard_normal((cfg.n_kv_heads, cfg.n_refs, cfg.head_dim))
    return (r / math.sqrt(cfg.head_dim)).astype(np.float32)


def scales(cfg: Config) -> np.ndarray:
    """Per-(sequence, KV head) key scale [B][Hkv]."""
    if not cfg.head_scale:
        return np.ones((cfg.batch, cfg.n_kv_heads), dtype=np.float64)
    return _rng(cfg, 1).uniform(0.5, 2.0, (cfg.batch, cfg.n_kv_heads))


def queries(cfg: Config, n: int | None = None) -> np.ndarray:
    """Decode queries [T][B][Hq][d] in the storage dtype (values widened to fp32).

    Queries arrive pre-scaled (entries ~ N(0, 1/d)), so the logit scale is 1.
    `n` limits the draw to the first n steps (the same values as a full draw).
    """
    T = cfg.n_queries if n is None else min(n, cfg.n_queries)
    shape = (cfg.batch, cfg.n_q_heads, cfg.head_dim)
    g = _rng(cfg, 3)
    per_step = int(np.prod(shape))
    q = g.standard_normal(T * per_step, dtype=np.float32).reshape((T,) + shape)
    return _store(cfg, q / np.float32(math.sqrt(cfg.head_dim)))


def needles(cfg: Config, b: int, g: int):
    """Planted needles of unit (b, g): arrays (t, h, pos), positions distinct in [1, N)."""
    rng = _rng(cfg, 4, b, g)
    G = cfg.group
    if cfg.needles_per_query:
        n = cfg.needles_per_query * cfg.n_queries
        t = np.repeat(np.arange(cfg.n_queries), cfg.needles_per_query)
        h = g * G + rng.integers(0, G, n)
    else:
        n = cfg.needles_per_unit
        t = rng.integers(0, cfg.n_queries, n)
        h = g * G + rng.integers(0, G, n)
    pos = 1 + rng.choice(cfg.n_tokens - 1, size=n, replace=False)
    return t.astype(np.int64), h.astype(np.int64), pos.astype(np.int64)


def unit_kv(cfg: Config, b: int, g: int, q: np.ndarray | None = None):
    """Keys and values of unit (b, g): two fp32 arrays [N][d] holding stored-dtype values."""
    N, d = cfg.n_tokens, cfg.head_dim
    s = np.float32(scales(cfg)[b, g])
    rng = _rng(cfg, 2, b, g)
    K = rng.standard_normal((N, d), dtype=np.float32)
    K *= s
    V = rng.standard_normal((N, d), dtype=np.float32)
    t, h, pos = needles(cfg, b, g)
    if len(pos):
        if q is None or q.shape[0] <= int(t.max()):
            q = queries(cfg, int(t.max()) + 1)
        qv = q[t, b, h].astype(np.float64)
        qhat = qv / np.linalg.norm(qv, axis=1, keepdims=True)
        K[pos] = (float(s) * 4.0 * qhat).astype(np.float32)
    return _store(cfg, K), _store(cfg, V)


def append_rows(cfg: Config, b: int, g: int):
    """Rows appended to unit (b, g) during decode: (K_new, V_new), each [append_steps][d]."""
    n, d = cfg.append_steps, cfg.head_dim
    s = np.float32(scales(cfg)[b, g])
    rng = _rng(cfg, 5, b, g)
    K = rng.standard_normal((n, d), dtype=np.float32) * s
    V = rng.standard_normal((n, d), dtype=np.float32)
    return _store(cfg, K), _store(cfg, V)
