"""Seeded synthetic inputs shared by the tests, the bench and the oracle runs.

This module only draws random numbers with a stated structure.  It holds none
of the compression method's arithmetic (no projection, no SVD, no RoPE, no
attention), so the oracle and the GPU path can both be fed from it without
sharing any of the method's code.

The pages' own workloads (reasoning traces of 8B models on MATH-500 / AIME)
are not available; these generators stand in for the structure the pages rely
on: keys and values that are strongly low-rank [iS-KV explainer, Jargon
"Low-rank" and the re-attention paragraph], plus a set of old tokens that later
queries attend to strongly (the re-attention statistic of the same paragraph).

Every stream is reproducible from (seed, sequence, layer, kv head, K|V) alone
through numpy's SeedSequence, so any unit can be regenerated independently.
"""

from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np


@dataclass(frozen=True)
class Workload:
    """Shapes and value model of one synthetic workload."""
    name: str
    batch: int
    kv_heads: int
    q_heads: int
    head_dim: int
    rank: int
    window: int
    context: int                # tokens in the cache at the measured decode step
    storage: str                # "bf16" or "f32"
    signal_rank: int
    noise_std: float
    spectrum: str = "gauss"     # "gauss" (flat Gaussian factors) or "power" (sigma_i ~ 1/i)
    num_layers: int = 1
    hot_fraction: float = 0.0   # share of positions given a high-norm aligned key
    hot_alpha: float = 4.0      # hot key norm, in units of the RMS key norm
    hot_beta: float = 2.0       # query alignment to the hot direction
    seed: int = 1000
    # True: the KV heads of a (sequence, layer) mix the same latent z_t (each
    # through its own G), so their rows side by side have rank signal_rank --
    # the structure a basis over all heads of a layer compresses
    shared_latent: bool = False
    extra: dict = field(default_factory=dict)


# The five workloads; sizes follow the stated configurations.  Config 4's query
# head count (32) is a reading: only "36 layers x 8 KV heads" is stated.
WORKLOADS = {
    1: Workload("1 KV head, r=32, 4096 past tokens, window 256, fp32",
                batch=1, kv_heads=1, q_heads=1, head_dim=128, rank=32, window=256,
                context=4096, storage="f32", signal_rank=24, noise_std=0.01, seed=1001),
    2: Workload("GQA layer 8 KV / 32 q heads, r=32, 32K context, window 256, bf16, batch 1",
                batch=1, kv_heads=8, q_heads=32, head_dim=128, rank=32, window=256,
                context=32768, storage="bf16", signal_rank=32, noise_std=0.01, seed=1002),
    3: Workload("batch 16 x 16K, 8 KV / 32 q heads, r=64, window 512, bf16, sigma_i ~ 1/i",
                batch=16, kv_heads=8, q_heads=32, head_dim=128, rank=64, window=512,
                context=16384, storage="bf16", signal_rank=128, noise_std=0.0,
                spectrum="power", seed=1003),
    4: Workload("36 layers x 8 KV / 32 q heads, r=32, window 1024, grown 4K to 64K, bf16",
                batch=1, kv_heads=8, q_heads=32, head_dim=128, rank=32, window=1024,
                context=65536, storage="bf16", signal_rank=32, noise_std=0.01,
                num_layers=36, hot_fraction=0.3, seed=1004),
    5: Workload("batch 64 x 8K, 8 KV / 32 q heads, r in {16,32,64,128} x window in {128,1024}, bf16",
                batch=64, kv_heads=8, q_heads=32, head_dim=128, rank=32, window=128,
                context=8192, storage="bf16", signal_rank=32, noise_std=0.01, seed=1005),
}


def with_(w: Workload, **kw) -> Workload:
    """Copy of a workload with some fields replaced (smaller test sizes etc.)."""
    d = dict(w.__dict__)
    d.update(kw)
    return Workload(**d)


def _rng(w: Workload, *key) -> np.random.Generator:
    return np.random.default_rng(np.random.SeedSequence([w.seed, *[int(k) for k in key]]))


def _haar(rng, n):
    """Haar-distributed orthogonal matrix (QR of a Gaussian, signs fixed)."""
    z = rng.standard_normal((n, n))
    q, r = np.linalg.qr(z)
    return q * np.sign(np.diag(r))


def unit_factors(w: Workload, b: int, layer: int, head: int, which: int):
    """Fixed per-unit mixing matrix G (d x k) and per-token scales (k,).

    which: 0 for keys, 1 for values.
    """
    rng = _rng(w, 0, b, layer, head, which)
    d, k = w.head_dim, w.signal_rank
    if w.spectrum == "gauss":
        g = rng.standard_normal((d, k)) / np.sqrt(k)      # unit variance entries
        scales = np.ones(k)
    elif w.spectrum == "power":
        o = _haar(rng, d)[:, :k]
        scales = 1.0 / np.arange(1, k + 1)
        scales = scales * np.sqrt(d / np.sum(scales ** 2))  # unit mean entry variance
        g = o
    else:
        raise ValueError(w.spectrum)
    return g, scales


def hot_direction(w: Workload, layer: int, head: int) -> np.ndarray:
    """Unit vector shared by the hot keys and the later queries of one KV head."""
    rng = _rng(w, 3, layer, head)
    u = rng.standard_normal(w.head_dim)
    return u / np.linalg.norm(u)


def unit_tokens(w: Workload, b: int, layer: int, head: int, which: int,
                start: int, count: int) -> np.ndarray:
    """Rows start..start+count-1 of one unit's K (which=0) or V (which=1) stream.

    x_t = G diag(scales) z_t + e_t, z_t ~ N(0, I_k), e_t ~ N(0, noise_std^2 I_d)
    (z_t common to the heads of the sequence and layer when shared_latent);
    with hot_fraction > 0, a seeded Bernoulli share of key positions also gets
    + alpha * sqrt(d) * u (u = hot_direction).  Rows are drawn per 64-token
    chunk, so any window of positions can be regenerated on its own.
    """
    g, scales = unit_factors(w, b, layer, head, which)
    d, k = w.head_dim, w.signal_rank
    out = np.empty((count, d))
    chunk = 64
    first = start // chunk
    last = (start + count - 1) // chunk if count else first - 1
    for c in range(first, last + 1):
        rng = _rng(w, 1, b, layer, head, which, c)
        if w.shared_latent:
            # z from a stream without the head; noise and hot keys per head
            z = _rng(w, 5, b, layer, which, c).standard_normal((chunk, k))
        else:
            z = rng.standard_normal((chunk, k))
        x = (z * scales) @ g.T
        if w.noise_std:
            x = x + w.noise_std * rng.standard_normal((chunk, d))
        if which == 0 and w.hot_fraction > 0:
            hot = rng.random(chunk) < w.hot_fraction
            x = x + np.outer(hot, w.hot_alpha * np.sqrt(d) * hot_direction(w, layer, head))
        lo = max(start, c * chunk)
        hi = min(start + count, (c + 1) * chunk)
        out[lo - start: hi - start] = x[lo - c * chunk: hi - c * chunk]
    return out


def tokens(w: Workload, layer: int, start: int, count: int) -> tuple[np.ndarray, np.ndarray]:
    """k, v of shape [batch, count, kv_heads, d] (float64) for one layer."""
    k = np.empty((w.batch, count, w.kv_heads, w.head_dim))
    v = np.empty_like(k)
    for b in range(w.batch):
        for h in range(w.kv_heads):
            k[b, :, h] = unit_tokens(w, b, layer, h, 0, start, count)
            v[b, :, h] = unit_tokens(w, b, layer, h, 1, start, count)
    return k, v


def query(w: Workload, layer: int, step: int) -> np.ndarray:
    """q of shape [batch, q_heads, d] (float64): N(0, I), plus beta * u for
    workloads with hot keys (u of the query head's KV head)."""
    rng = _rng(w, 2, layer, step)
    q = rng.standard_normal((w.batch, w.q_heads, w.head_dim))
    if w.hot_fraction > 0:
        g = w.q_heads // w.kv_heads
        for hq in range(w.q_heads):
            q[:, hq] += w.hot_beta * hot_direction(w, layer, hq // g)
    return q


def _bf16_grid(x: np.ndarray) -> np.ndarray:
    """float32 values with the low 16 mantissa bits cleared, so that they are
    exactly representable in bfloat16 (truncation: a way to draw values on the
    bf16 grid, not a model of any store)."""
    u = np.asarray(x, dtype=np.float32).view(np.uint32) & np.uint32(0xFFFF0000)
    return u.view(np.float32)


def synthetic_unit(w: Workload, b: int, h: int, length: int, n_c: int, max_tokens: int,
                   seed: int = 7, rank_v: int = 0, ring_in_span: bool = False):
    """One (sequence b, KV head h) of a random cache state of the workload's
    shapes, for checks at full size without running the folds that would build
    it: per K|V an orthonormal d x r basis (QR of a Gaussian matrix), singular
    values, coefficient rows [0, n_c) and ring rows for the exact positions
    [n_c, length) at slot p mod (window + 64).  With bf16 storage the
    coefficients and ring rows are drawn on the bf16 grid.  ring_in_span: ring
    rows lie in the span of the basis (plus 1e-3 noise), so that a fold of the
    state has a well separated rank-r truncation.

    Returns [K, V] dicts with keys basis, S, coef (max_tokens x r), ring
    ((window + 64) x d).  rank_v > 0 gives the V factor that rank instead of
    w.rank."""
    d, slots = w.head_dim, w.window + 64
    assert n_c % 64 == 0 and w.window <= length - n_c <= w.window + 64
    xs = []
    for x in range(2):
        r = (rank_v or w.rank) if x else w.rank
        rng = _rng(w, 9001, seed, b, h, x)          # 9001: state stream tag
        B, _ = np.linalg.qr(rng.standard_normal((d, r)))
        S = np.sort(rng.uniform(1.0, 50.0, r))[::-1].astype(np.float32)
        C = np.zeros((max_tokens, r), np.float32)
        C[:n_c] = rng.standard_normal((n_c, r)).astype(np.float32) * (2.0 / np.sqrt(r))
        ring = np.zeros((slots, d), np.float32)
        pos = np.arange(n_c, length)
        if ring_in_span:
            z = rng.standard_normal((len(pos), r)) * (2.0 / np.sqrt(r))
            rows = z @ B.T + 1e-3 * rng.standard_normal((len(pos), d))
        else:
            rows = rng.standard_normal((len(pos), d)) * 0.25
        ring[pos % slots] = rows.astype(np.float32)
        if w.storage == "bf16":
            C, ring = _bf16_grid(C), _bf16_grid(ring)
        xs.append(dict(basis=B.astype(np.float32), S=S, coef=C, ring=ring))
    return xs


def synthetic_state(w: Workload, length: int, n_c: int, max_tokens: int, seed: int = 7,
                    rank_v: int = 0, ring_in_span: bool = False):
    """synthetic_unit for every (sequence, KV head), as a list over units
    (b * kv_heads + h)."""
    return [synthetic_unit(w, b, h, length, n_c, max_tokens, seed, rank_v, ring_in_span)
            for b in range(w.batch) for h in range(w.kv_heads)]


def synthetic_joint(w: Workload, b: int, length: int, n_c: int, max_tokens: int, seed: int = 7,
                    rank_v: int = 0, ring_in_span: bool = False):
    """synthetic_unit for a joint basis over the kv_heads heads of sequence b:
    per K|V an orthonormal (kv_heads*d x r) basis, singular values, one
    coefficient row per position for all heads, and ring rows of all heads
    side by side ((window + 64) x kv_heads*d)."""
    D, slots = w.kv_heads * w.head_dim, w.window + 64
    assert n_c % 64 == 0 and w.window <= length - n_c <= w.window + 64
    xs = []
    for x in range(2):
        r = (rank_v or w.rank) if x else w.rank
        rng = _rng(w, 9002, seed, b, x)             # 9002: joint state stream tag
        B, _ = np.linalg.qr(rng.standard_normal((D, r)))
        S = np.sort(rng.uniform(1.0, 50.0, r))[::-1].astype(np.float32)
        C = np.zeros((max_tokens, r), np.float32)
        C[:n_c] = rng.standard_normal((n_c, r)).astype(np.float32) * (2.0 / np.sqrt(r))
        ring = np.zeros((slots, D), np.float32)
        pos = np.arange(n_c, length)
        if ring_in_span:
            z = rng.standard_normal((len(pos), r)) * (2.0 / np.sqrt(r))
            rows = z @ B.T + 1e-3 * rng.standard_normal((len(pos), D))
        else:
            rows = rng.standard_normal((len(pos), D)) * 0.25
        ring[pos % slots] = rows.astype(np.float32)
        if w.storage == "bf16":
            C, ring = _bf16_grid(C), _bf16_grid(ring)
        xs.append(dict(basis=B.astype(np.float32), S=S, coef=C, ring=ring))
    return xs
