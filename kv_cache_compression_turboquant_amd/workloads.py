"""Seeded synthetic inputs for the TurboQuant workloads (numpy only; none of the method's
arithmetic lives here).  Both the HIP path and the CPU oracle are fed the arrays made here.

The pages measure on real model KV caches and public benchmarks that are not available; these
generators stand in for them with the shapes the pages give (head_dim 128, GQA, d up to 3072):

* keys: i.i.d. N(0, 1) entries; per kv head, 4 distinct "outlier" channels (drawn without
  replacement) scaled x8; each (sequence, head, token) vector multiplied by a LogNormal(0, 0.5)
  factor; rounded to bf16 (round to nearest even).
* values: N(0, 1) with 4 outlier channels x8 per kv head, no per-token factor, bf16.
* queries: N(0, 1) fp32.
* vector index: x = g + sqrt(beta) U w (rank-64 component U orthonormal), normalised to unit
  length; queries from the same law.
"""

from dataclasses import dataclass, field

import numpy as np

D_HEAD = 128


def f32_to_bf16_bits(a):
    """Round fp32 to bf16 (nearest even) and return the 16-bit patterns (uint16)."""
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)
    u = u + (np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1)))
    return (u >> np.uint32(16)).astype(np.uint16)


def bf16_bits_to_f32(h):
    return (np.asarray(h, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def gaussian(shape, seed):
    return np.random.default_rng(seed).standard_normal(shape, dtype=np.float32)


def outlier_channels(hkv, d, seed, count=4):
    rng = np.random.default_rng(seed)
    return np.stack([rng.choice(d, size=count, replace=False) for _ in range(hkv)])


def kv_tensor_bf16(B, hkv, T, d, seed, outlier_seed, scale_seed=None, outlier_scale=8.0,
                   lognormal_sigma=0.5):
    """[B, hkv, T, d] bf16 bit patterns (uint16), generated one (b, head) slab at a time."""
    out = np.empty((B, hkv, T, d), dtype=np.uint16)
    chans = outlier_channels(hkv, d, outlier_seed)
    g = np.random.default_rng(seed)
    s = np.random.default_rng(scale_seed) if scale_seed is not None else None
    for b in range(B):
        for h in range(hkv):
            slab = g.standard_normal((T, d), dtype=np.float32)
            slab[:, chans[h]] *= np.float32(outlier_scale)
            if s is not None:
                lam = s.lognormal(0.0, lognormal_sigma, size=T).astype(np.float32)
                slab *= lam[:, None]
            out[b, h] = f32_to_bf16_bits(slab)
    return out


def iter_lowrank_unit_vectors(n, d, rank, beta, seed_g, seed_u, seed_w, chunk=65536):
    """Yields (first row, rows) of n unit vectors g + sqrt(beta) U w, normalised, in chunks;
    U = Q factor of a seeded Gaussian [d, rank]."""
    u, _ = np.linalg.qr(np.random.default_rng(seed_u).standard_normal((d, rank)))
    rg = np.random.default_rng(seed_g)
    rw = np.random.default_rng(seed_w)
    for lo in range(0, n, chunk):
        hi = min(n, lo + chunk)
        g = rg.standard_normal((hi - lo, d))
        w = rw.standard_normal((hi - lo, rank))
        x = g + np.sqrt(beta) * (w @ u.T)
        x /= np.linalg.norm(x, axis=1, keepdims=True)
        yield lo, x.astype(np.float32)


def lowrank_unit_vectors(n, d, rank, beta, seed_g, seed_u, seed_w, chunk=65536):
    """n unit vectors g + sqrt(beta) U w (fp32 [n, d]), normalised; U = Q factor of a seeded Gaussian."""
    out = np.empty((n, d), dtype=np.float32)
    for lo, x in iter_lowrank_unit_vectors(n, d, rank, beta, seed_g, seed_u, seed_w, chunk):
        out[lo:lo + x.shape[0]] = x
    return out


@dataclass(frozen=True)
class Config:
    name: str
    workload: str
    d: int
    bits: int
    mode: str
    B: int = 1
    hkv: int = 1
    hq: int = 1
    T: int = 0
    n: int = 0
    rot_seed: int = 1
    qjl_seed: int = 2
    extra: dict = field(default_factory=dict)


CONFIGS = {
    "c1": Config("c1", "tiny MSE round trip: 4096 fp32 N(0,1) vectors, d=128, b=2, 32 queries",
                 d=128, bits=2, mode="mse", B=1, hkv=1, hq=32, T=4096, n=4096),
    "c2": Config("c2", "single-layer KV-key compression, Llama-3-8B shape: 1 x 8 KV heads x 32768 "
                 "tokens x d=128 bf16, MSE b=3 encode + decode-step scores of 32 query heads",
                 d=128, bits=3, mode="mse", B=1, hkv=8, hq=32, T=32768),
    "c3": Config("c3", "TurboQuant_prod b=4: 16 x 16384 tokens x 8 KV heads x d=128 bf16, "
                 "unbiased scores of 32 query heads", d=128, bits=4, mode="prod", B=16, hkv=8,
                 hq=32, T=16384),
    "c4": Config("c4", "fused compressed decode attention: 4 x 131072 tokens x 8 KV heads, d=128, "
                 "K and V MSE", d=128, bits=2, mode="mse", B=4, hkv=8, hq=32, T=131072),
    "c5": Config("c5", "vector index: 1e6 unit vectors d=1536, prod b=4, 1024 queries, top-10",
                 d=1536, bits=4, mode="prod", n=1_000_000, extra={"queries": 1024, "k": 10}),
}


def c1_inputs():
    return gaussian((4096, 128), 0), gaussian((32, 128), 2)


def kv_keys(cfg, T=None, B=None):
    """Keys of a KV config (bf16 bits [B, hkv, T, d]) with seeds 0 (values), 10 (outlier
    channels), 11 (per-token scale)."""
    return kv_tensor_bf16(B or cfg.B, cfg.hkv, T or cfg.T, cfg.d, seed=0, outlier_seed=10, scale_seed=11)


def kv_values(cfg, T=None, B=None):
    return kv_tensor_bf16(B or cfg.B, cfg.hkv, T or cfg.T, cfg.d, seed=20, outlier_seed=21, scale_seed=None)


def index_vectors(cfg):
    """Database generator of the vector-index workload (seeds 0 / 30 / 31, beta 24, rank 64)."""
    return iter_lowrank_unit_vectors(cfg.n, cfg.d, 64, 24.0, 0, 30, 31)


def index_queries(cfg):
    """The workload's queries: the same law, seeds 32 / 30 / 33."""
    return lowrank_unit_vectors(cfg.extra["queries"], cfg.d, 64, 24.0, 32, 30, 33)


def kv_queries(cfg, B=None):
    return gaussian((B or cfg.B, cfg.hq, cfg.d), 12)
