"""Seeded synthetic inputs (NumPy, fp16) shared by the tests, the benchmark
and the oracle checks.  This module holds no codec arithmetic: it only draws
K/V caches and queries of the shapes and value distributions of the
workloads below.

  tiny        1 layer, 1 KV head, head_dim 128, 1024 tokens; K, V ~ N(0,1)
              with 4 outlier channels scaled x20; one N(0,1) query.
  llama8b     32 query / 8 KV heads (GQA 4), 32768 tokens, batch 1; K =
              lognormal(0, 0.5) per-(head, channel) scale x Student-t(3)
              noise; V ~ N(0,1); queries N(0,1).
  minmax      32 layers x 8 KV heads x 128 x 4096 tokens, K and V; N(0,1)
              times a per-64-group scale drawn log-uniform in [1e-3, 8].
  llama70b    80 layers, 8 KV heads, 64 query heads, 131072 tokens; each
              layer's K/V drawn like `tiny` from seed 404 + layer.
  needle      64 sequences x 8192 tokens, 32 query / 8 KV heads; K ~ N(0,1)
              with 8 outlier channels x20 per KV head, V ~ N(0,1); 16 needle
              positions per sequence; query head h points at needle h mod 16
              of its KV head (outlier channels removed), scaled to norm
              3*sqrt(128), so each head's softmax is dominated by one token.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field

import numpy as np

D = 128


@dataclass
class AttnCase:
    name: str
    k: np.ndarray          # [B, Hkv, T, D] fp16
    v: np.ndarray          # [B, Hkv, T, D] fp16
    q: np.ndarray          # [B, Hq, D] fp16
    seq_lens: np.ndarray | None = None
    meta: dict = field(default_factory=dict)

    @property
    def shape(self):
        B, Hkv, T, _ = self.k.shape
        return B, self.q.shape[1], Hkv, T


def _outlier_normal(rng, shape, n_out, scale=20.0):
    """N(0,1) over [..., T, D] with n_out channels (per leading index) x scale."""
    x = rng.standard_normal(shape, dtype=np.float32)
    lead = int(np.prod(shape[:-2])) if len(shape) > 2 else 1
    xr = x.reshape(lead, shape[-2], shape[-1])
    for i in range(lead):
        ch = rng.choice(shape[-1], n_out, replace=False)
        xr[i][:, ch] *= scale
    return x


def tiny(seed: int = 101, T: int = 1024) -> AttnCase:
    rng = np.random.default_rng(seed)
    k = _outlier_normal(rng, (T, D), 4).reshape(1, 1, T, D)
    v = _outlier_normal(rng, (T, D), 4).reshape(1, 1, T, D)
    q = rng.standard_normal((1, 1, D), dtype=np.float32)
    return AttnCase("tiny", k.astype(np.float16), v.astype(np.float16), q.astype(np.float16),
                    meta={"kf": ("prod", 2), "vf": ("mse", 2), "tau": 1e-6})


def llama8b(seed: int = 202, T: int = 32768, Hq: int = 32, Hkv: int = 8, B: int = 1) -> AttnCase:
    rng = np.random.default_rng(seed)
    s = rng.lognormal(0.0, 0.5, (B, Hkv, 1, D)).astype(np.float32)
    eps = rng.standard_t(3, (B, Hkv, T, D)).astype(np.float32)
    k = s * eps
    v = rng.standard_normal((B, Hkv, T, D), dtype=np.float32)
    q = rng.standard_normal((B, Hq, D), dtype=np.float32)
    return AttnCase("llama8b", k.astype(np.float16), v.astype(np.float16), q.astype(np.float16),
                    meta={"kf": ("prod", 3), "vf": ("mse", 4), "tau": 1e-6})


def minmax_tensor(seed: int = 303, layers: int = 32, heads: int = 8, tokens: int = 4096,
                  group: int = 64) -> np.ndarray:
    """One tensor (K or V) of the min-max workload, flattened fp16."""
    rng = np.random.default_rng(seed)
    n = layers * heads * tokens * D
    x = rng.standard_normal(n, dtype=np.float32).reshape(-1, group)
    x *= np.exp(rng.uniform(math.log(1e-3), math.log(8.0), (x.shape[0], 1))).astype(np.float32)
    return x.reshape(-1).astype(np.float16)


BOUNDARY_LAYERS_70B = (0, 1, 78, 79)


def llama70b_layer(layer: int, T: int = 131072, Hkv: int = 8, Hq: int = 64) -> AttnCase:
    rng = np.random.default_rng(404 + layer)
    k = _outlier_normal(rng, (Hkv, T, D), 4).reshape(1, Hkv, T, D)
    v = _outlier_normal(rng, (Hkv, T, D), 4).reshape(1, Hkv, T, D)
    q = rng.standard_normal((1, Hq, D), dtype=np.float32)
    boundary = layer in BOUNDARY_LAYERS_70B
    fm = ("q8", 8) if boundary else None
    return AttnCase(f"llama70b.l{layer}", k.astype(np.float16), v.astype(np.float16), q.astype(np.float16),
                    meta={"kf": fm or ("prod", 2), "vf": fm or ("mse", 2), "tau": 1e-6, "layer": layer})


def needle(seed: int = 505, B: int = 64, T: int = 8192, Hq: int = 32, Hkv: int = 8,
           n_needles: int = 16) -> AttnCase:
    rng = np.random.default_rng(seed)
    k = rng.standard_normal((B, Hkv, T, D), dtype=np.float32)
    out_ch = np.stack([rng.choice(D, 8, replace=False) for _ in range(Hkv)])  # [Hkv, 8]
    for h in range(Hkv):
        k[:, h][:, :, out_ch[h]] *= 20.0
    v = rng.standard_normal((B, Hkv, T, D), dtype=np.float32)
    k16 = k.astype(np.float16)
    g = Hq // Hkv
    needles = np.stack([np.sort(rng.choice(T, n_needles, replace=False)) for _ in range(B)])  # [B, 16]
    q = np.zeros((B, Hq, D), np.float32)
    for b in range(B):
        for h in range(Hq):
            kvh = h // g
            kn = k16[b, kvh, needles[b, h % n_needles]].astype(np.float32).copy()
            kn[out_ch[kvh]] = 0.0
            q[b, h] = 3.0 * math.sqrt(D) * kn / np.linalg.norm(kn)
    return AttnCase("needle", k16, v.astype(np.float16), q.astype(np.float16),
                    meta={"kf": ("prod", 3), "vf": ("mse", 2), "tau": 1e-6, "needles": needles})


def slice_case(c: AttnCase, B: int | None = None, Hkv: int | None = None, T: int | None = None) -> AttnCase:
    """A smaller case cut from a larger one (same value distribution)."""
    B0, Hq0, Hkv0, T0 = c.shape
    B = B or B0
    Hkv = Hkv or Hkv0
    T = T or T0
    g = Hq0 // Hkv0
    return AttnCase(c.name + ".slice", np.ascontiguousarray(c.k[:B, :Hkv, :T]),
                    np.ascontiguousarray(c.v[:B, :Hkv, :T]), np.ascontiguousarray(c.q[:B, :Hkv * g]),
                    None if c.seq_lens is None else c.seq_lens[:B], dict(c.meta))
