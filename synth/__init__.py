"""Seeded synthetic inputs for the five workloads.

This module holds no arithmetic of the compression method: it draws the vectors the
method is applied to (K, V, queries, database vectors), applies the model-side RoPE that
precedes the method, and names the seeds of the codec's random matrices.  Both the HIP
path and the CPU oracle receive exactly these arrays.

Workloads (shapes and distributions follow the pages' settings; the data are synthetic
stand-ins since no model weights or datasets are used):

1. tiny         1 head, d = 64, 256 keys/values, 1 query, fp32 N(0, 1) from seed 0.
2. esm2         ESM-2-650M-shaped cache: 33 layers x 20 heads, d = 64, 1024 tokens, fp16;
                20 prototype vectors (the amino-acid vocabulary) plus noise, 4 channels
                per head scaled 20x, RoPE (base 10000) on keys and on the query.
3. gqa_decode   8B-class GQA decode: 32 layers, 32 query / 8 KV heads, d = 128, batch 8,
                32768 cached tokens, bf16 N(0, 1) with 2% of channels scaled 10x.
4. long_ctx     as 3 with batch 1 and 131072 tokens.
5. search       1,000,000 x 200 unit vectors from a 1000-component Gaussian mixture,
                10,000 queries from the same mixture.
"""

from dataclasses import dataclass

import numpy as np

# Codec seeds (SplitMix64 stream seeds) shared by every workload.
SEED_ROT_K = 1
SEED_SKETCH_K = 2
SEED_ROT_V = 3
SEED_SKETCH_V = 4


def esm2_basis_seed(layer: int, head: int) -> int:
    """Seed of the optional per-(layer, head) orthogonal basis composed before Pi."""
    return (2 << 32) | (layer << 16) | head


@dataclass(frozen=True)
class Workload:
    name: str
    layers: int
    batch: int
    hq: int
    hkv: int
    d: int
    n_ctx: int
    k_bits: int
    k_m: int
    v_bits: int
    v_m: int

    @property
    def n_seq(self) -> int:
        return self.layers * self.batch

    @property
    def group(self) -> int:
        return self.hq // self.hkv


TINY = Workload("tiny", 1, 1, 1, 1, 64, 256, 2, 64, 2, 64)
ESM2 = Workload("esm2_650m", 33, 1, 20, 20, 64, 1024, 3, 64, 3, 64)
GQA_DECODE = Workload("gqa8b_decode_b8_32k", 32, 8, 32, 8, 128, 32768, 2, 128, 3, 0)
LONG_CTX = Workload("gqa8b_decode_b1_128k", 32, 1, 32, 8, 128, 131072, 2, 128, 3, 0)
SEARCH_D, SEARCH_BITS, SEARCH_M = 200, 2, 200
SEARCH_N_DB, SEARCH_N_Q, SEARCH_CLUSTERS = 1_000_000, 10_000, 1000


def scaled(w: Workload, layers=None, batch=None, n_ctx=None) -> Workload:
    """The same workload with fewer layers, sequences or tokens (test-size cases)."""
    return Workload(w.name + "_slice", layers or w.layers, batch or w.batch, w.hq, w.hkv, w.d,
                    n_ctx or w.n_ctx, w.k_bits, w.k_m, w.v_bits, w.v_m)


# ------------------------------------------------------------------------------- 1


def tiny():
    """K [256, 64], V [256, 64], q [64], fp32 N(0, 1), drawn in that order from seed 0."""
    g = np.random.default_rng(0)
    k = g.standard_normal((256, 64)).astype(np.float32)
    v = g.standard_normal((256, 64)).astype(np.float32)
    q = g.standard_normal(64).astype(np.float32)
    return k, v, q


# ------------------------------------------------------------------------------- 2


def rope(x: np.ndarray, pos: np.ndarray, base: float = 10000.0) -> np.ndarray:
    """Rotary position embedding on the last axis, half-split pairs (i, i + d/2), in fp64."""
    x = np.asarray(x, dtype=np.float64)
    d = x.shape[-1]
    half = d // 2
    theta = np.asarray(pos, dtype=np.float64)[..., None] * base ** (-2.0 * np.arange(half) / d)
    c, s = np.cos(theta), np.sin(theta)
    a, b = x[..., :half], x[..., half:]
    return np.concatenate([a * c - b * s, a * s + b * c], axis=-1)


def esm2(layers: int = 33, heads: int = 20, seq: int = 1024, d: int = 64, noise: float = 0.1):
    """K, V [layers, heads, seq, d] fp16 (K RoPE'd) and q [layers, heads, d] fp32 (RoPE'd at seq)."""
    letters = np.random.default_rng(1).integers(0, 20, seq)
    K = np.empty((layers, heads, seq, d), np.float16)
    V = np.empty((layers, heads, seq, d), np.float16)
    q = np.empty((layers, heads, d), np.float32)
    pos = np.arange(seq)
    for l in range(layers):
        for h in range(heads):
            g = np.random.default_rng(np.random.SeedSequence([1, l, h]))
            ek = g.standard_normal((20, d))
            ev = g.standard_normal((20, d))
            kx = ek[letters] + noise * g.standard_normal((seq, d))
            vx = ev[letters] + noise * g.standard_normal((seq, d))
            kx[:, g.choice(d, 4, replace=False)] *= 20.0
            vx[:, g.choice(d, 4, replace=False)] *= 20.0
            K[l, h] = rope(kx, pos).astype(np.float16)
            V[l, h] = vx.astype(np.float16)
            q[l, h] = rope(g.standard_normal(d), np.array(seq)).astype(np.float32)
    return K, V, q


# ------------------------------------------------------------------------------- 3, 4


def gqa_outlier_channels(w: Workload, seed: int, layers=None):
    """The 10x channels: [layers, hkv, 2 (K, V), round(0.02 d)] int64, from numpy seed ``seed``."""
    L = layers or w.layers
    n_out = int(round(0.02 * w.d))
    cg = np.random.default_rng(seed)
    out = np.empty((L, w.hkv, 2, n_out), np.int64)
    for l in range(L):
        for h in range(w.hkv):
            for t in range(2):
                out[l, h, t] = cg.choice(w.d, n_out, replace=False)
    return out


def gqa_decode(w: Workload, seed: int, device="cuda", layers=None):
    """K, V [layers, batch, hkv, n_ctx, d] bf16 and q [layers, batch, hq, d] fp32 (torch tensors).

    Drawn with a torch generator on ``device`` (so the values depend on the device type).
    Per (layer, kv head) the channels of ``gqa_outlier_channels`` are scaled 10x.  The data
    are taken as post-RoPE; queries are N(0, 1) without outliers.
    """
    import torch

    L = layers or w.layers
    gen = torch.Generator(device=device)
    gen.manual_seed(seed)
    shape = (L, w.batch, w.hkv, w.n_ctx, w.d)
    K = torch.randn(shape, generator=gen, device=device, dtype=torch.bfloat16)
    V = torch.randn(shape, generator=gen, device=device, dtype=torch.bfloat16)
    q = torch.randn((L, w.batch, w.hq, w.d), generator=gen, device=device, dtype=torch.float32)
    ch = gqa_outlier_channels(w, seed, L)
    for t, X in enumerate((K, V)):
        scale = torch.ones((L, w.hkv, w.d), dtype=torch.bfloat16)
        for l in range(L):
            for h in range(w.hkv):
                scale[l, h, ch[l, h, t]] = 10.0
        X.mul_(scale.to(device)[:, None, :, None, :])
    return K, V, q


# ------------------------------------------------------------------------------- 5


def search_data(n_db: int = SEARCH_N_DB, n_q: int = SEARCH_N_Q, d: int = SEARCH_D,
                clusters: int = SEARCH_CLUSTERS, sigma: float = 1.0):
    """Unit-normalised database [n_db, d] and queries [n_q, d] (fp32) from one Gaussian mixture."""
    g = np.random.default_rng(4)
    means = g.standard_normal((clusters, d))
    db = means[g.integers(0, clusters, n_db)]
    db += sigma * g.standard_normal((n_db, d))
    db /= np.linalg.norm(db, axis=1, keepdims=True)
    gq = np.random.default_rng(5)
    qs = means[gq.integers(0, clusters, n_q)] + sigma * gq.standard_normal((n_q, d))
    qs /= np.linalg.norm(qs, axis=1, keepdims=True)
    return db.astype(np.float32), qs.astype(np.float32)


# ------------------------------------------------------------------------------- misc


def pre_rotated(n: int, d: int, seed: int) -> np.ndarray:
    """fp32 N(0, 1) vectors standing for already-rotated inputs y (the rotated law of Gaussian data)."""
    return np.random.default_rng(seed).standard_normal((n, d)).astype(np.float32)


def random_codes(n: int, d: int, bits: int, m: int, idx_stride: int, sign_stride: int, seed: int):
    """Synthetic code planes (uniform index/sign bits, plausible fp16 norms) for scoring tests.

    Returns (idx uint8 [n, idx_stride], sign uint8 [n, sign_stride] or None, norms uint32 [n]);
    bits beyond the record and pad bytes are zero.  The norms are fp16 patterns of
    |N(0,1)| * sqrt(d) (key norm) and 0.35 |N(0,1)| * sqrt(d) (residual norm).
    """
    g = np.random.default_rng(seed)
    nb = d * bits
    idx = np.zeros((n, idx_stride), np.uint8)
    full, rem = divmod(nb, 8)
    idx[:, :full] = g.integers(0, 256, (n, full), dtype=np.uint8)
    if rem:
        idx[:, full] = g.integers(0, 1 << rem, n, dtype=np.uint8)
    sign = None
    if m > 0:
        sign = np.zeros((n, sign_stride), np.uint8)
        sf, sr = divmod(m, 8)
        sign[:, :sf] = g.integers(0, 256, (n, sf), dtype=np.uint8)
        if sr:
            sign[:, sf] = g.integers(0, 1 << sr, n, dtype=np.uint8)
    n16 = (np.abs(g.standard_normal(n)) * np.sqrt(d)).astype(np.float16).view(np.uint16).astype(np.uint32)
    r16 = (0.35 * np.abs(g.standard_normal(n)) * np.sqrt(d)).astype(np.float16).view(np.uint16).astype(np.uint32)
    return idx, sign, (r16 << 16) | n16
