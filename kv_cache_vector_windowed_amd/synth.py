"""Seeded synthetic inputs shared by the tests, the benchmark and the smoke check.

This module only draws inputs: it contains none of the method's arithmetic
(no second moment, no factorisation, no assignment, no selection, no rotation).
Both the GPU path and the CPU oracle consume exactly the arrays built here.

Recipe (stated once, used everywhere):

* Per (workload seed ``cfg``, head ``h``) the key distribution is a zero-mean
  Gaussian with per-channel variances ``s = 10**U(-1, 1)`` (log-uniform in
  [0.1, 10]) and four outlier channels whose values are multiplied by 20.
  ``s`` and the outlier channels come from stream 0.
* ``draw(n, stream)`` returns ``n`` fp32 rows of that distribution from the
  given stream.  Keys use stream 1, the codebook stream 2 (the first ``C`` rows
  of a separate seeded draw), decode-time new keys stream 6, value rows stream 8;
  the shared sub-vector codebook picks (stream 7) from pooled stream-2 sub-vectors.
* Calibration queries are ``G @ A.T`` with ``A ~ N(0, 1/d)`` (stream 3) and
  ``G ~ N(0, 1)`` of shape ``[M, d]`` (stream 4), i.e. Gaussian with the
  non-diagonal covariance ``A A^T``.
* Every generator is ``numpy.random.default_rng(SeedSequence([cfg, h, stream]))``.

The anisotropic variances and the outliers make the query-weighted objective
differ from plain nearest-centroid assignment, which is the case the pages'
query-aware quantiser is about.
"""
from __future__ import annotations

import dataclasses
from typing import Optional

import numpy as np

D = 128


def rng(cfg: int, h: int, stream: int) -> np.random.Generator:
    return np.random.default_rng(np.random.SeedSequence([int(cfg), int(h), int(stream)]))


def key_distribution(cfg: int, h: int, d: int = D):
    """Per-channel variances and the four outlier channels of head ``h``."""
    g = rng(cfg, h, 0)
    s = 10.0 ** g.uniform(-1.0, 1.0, d)
    outl = g.choice(d, size=min(4, d), replace=False)
    return s, outl


def draw(cfg: int, h: int, n: int, stream: int, d: int = D) -> np.ndarray:
    s, outl = key_distribution(cfg, h, d)
    g = rng(cfg, h, stream).standard_normal((n, d))
    x = g * np.sqrt(s)
    x[:, outl] *= 20.0
    return x.astype(np.float32)


# --------------------------------------------------------------------------- bf16 storage
def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round fp32 values to bf16 (round to nearest, ties to even); returns raw uint16."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    r = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return r.astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.ascontiguousarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


@dataclasses.dataclass
class Keys:
    """Keys of several heads: exact values as fp32 plus their storage form."""

    values: np.ndarray            # [heads, n, d] float32 (already bf16-exact for bf16 storage)
    dtype: str                    # "f32" or "bf16"
    bits: Optional[np.ndarray]    # [heads, n, d] uint16 raw bf16 bits, or None for f32


def keys(cfg: int, heads: int, n: int, dtype: str, d: int = D, stream: int = 1) -> Keys:
    vals = np.stack([draw(cfg, h, n, stream, d) for h in range(heads)])
    if dtype == "bf16":
        bits = f32_to_bf16_bits(vals)
        return Keys(bf16_bits_to_f32(bits), "bf16", bits)
    if dtype == "f32":
        return Keys(vals, "f32", None)
    raise ValueError(dtype)


def codebook(cfg: int, heads: int, c: int, d: int = D) -> np.ndarray:
    """[heads, c, d] fp32: the first ``c`` rows of a separate seeded key draw."""
    return np.stack([draw(cfg, h, c, 2, d) for h in range(heads)])


def queries(cfg: int, heads: int, m: int, d: int = D) -> np.ndarray:
    """[heads, m, d] fp32 Gaussian queries with covariance A A^T, A ~ N(0, 1/d)."""
    out = np.empty((heads, m, d), dtype=np.float32)
    for h in range(heads):
        a = rng(cfg, h, 3).standard_normal((d, d)) / np.sqrt(d)
        g = rng(cfg, h, 4).standard_normal((m, d))
        out[h] = (g @ a.T).astype(np.float32)
    return out


def new_keys(cfg: int, heads: int, n: int, d: int = D) -> np.ndarray:
    """Decode-time incoming keys, [heads, n, d] fp32 (stream 6)."""
    return np.stack([draw(cfg, h, n, 6, d) for h in range(heads)])


def uniform_codes(cfg: int, shape, c: int) -> np.ndarray:
    return rng(cfg, 0, 5).integers(0, c, size=shape).astype(np.uint16)


def pq_codebook(cfg: int, heads: int, k: int, sub_dim: int, d: int = D) -> np.ndarray:
    """[k, sub_dim] fp32 shared sub-vector codebook: k sub-vectors picked (stream 7) from the
    pooled sub-vectors of a separate seeded draw (stream 2) of every head, standing in for the
    pages' codebook trained on pooled calibration keys."""
    per = (k + heads - 1) // heads
    pool = np.concatenate([draw(cfg, h, per, 2, d).reshape(-1, sub_dim) for h in range(heads)])
    pick = rng(cfg, 0, 7).choice(pool.shape[0], size=k, replace=False)
    return np.ascontiguousarray(pool[pick])



# --------------------------------------------------------------------------- workloads
@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    cfg: int                 # seed index
    heads: int
    n: int                   # tokens (keys) per head and sequence
    c: int                   # centroids per head
    key_dtype: str           # "f32" / "bf16"
    m: int = 0               # calibration queries per head (0: no calibration)
    window: int = 0
    cur_pos: int = 0
    fraction: float = 0.0
    betas: tuple = ()
    batch: int = 1
    far_b: int = 2048
    rope_base: float = 10000.0
    dist: bool = False
    d: int = D
    q_heads: int = 0         # query heads per sequence sharing the key heads (0: heads)


WORKLOADS = {
    # Tiny single head, fp32 keys; every call.
    "tiny": Workload("tiny", 0, 1, 4096, 256, "f32", m=2048, window=64, cur_pos=4095,
                     fraction=0.1, betas=(1.0, 0.7)),
    # One Llama-3.2-3B-shaped layer: 8 KV heads x 32768 tokens, H-weighted encode then reconstruct.
    "layer": Workload("layer", 1, 8, 32768, 1024, "bf16", m=4096, window=512, cur_pos=32767,
                      fraction=0.1),
    # Decode-step re-expansion: 32 sequences x 8 heads x 16384 tokens, fp32 output,
    # plus a cosine-blend assignment of the one new key per (sequence, head).
    "decode": Workload("decode", 2, 8, 16384, 1024, "f32", window=256, cur_pos=16384,
                       betas=(0.8,), batch=32),
    # Large-codebook encode stress: 8 x 131072 bf16 keys, C = 4096, codes + distances.
    "encode_stress": Workload("encode_stress", 3, 8, 131072, 4096, "bf16", m=8192, dist=True),
    # Long-context pipeline: 8 x 131072 bf16, 5% retrieval split, C = 2048, W = 1024.
    "long_context": Workload("long_context", 4, 8, 131072, 2048, "bf16", m=4096, window=1024,
                             cur_pos=131071, fraction=0.05),
    # Top-K retrieval over codes on the decode shape: 32 sequences x 24 query heads over 8 key
    # heads (Llama-3.2-3B grouping) x 16384 codes uniform over C = 1024; k = 10% of the tokens.
    "topk_decode": Workload("topk_decode", 2, 8, 16384, 1024, "f32", fraction=0.1, batch=32,
                            q_heads=24),
    # The pages' default configuration on the layer shape: sub-vector codes (sub_dim 8, one
    # shared codebook of 2^8 entries), W = 128, retrieval fraction 0.2, beta 0.5; keys and
    # values, 8 heads x 32768 bf16 tokens.  c is the codebook size k.
    "pq_layer": Workload("pq_layer", 5, 8, 32768, 256, "bf16", m=4096, window=128,
                         cur_pos=32767, fraction=0.2, betas=(0.5,)),
}
