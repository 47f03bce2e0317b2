"""Seeded synthetic inputs for the five block-sparse / top-k attention workloads.

This module only draws random numbers and lays out masks; it performs none of
the attention, planning or merge arithmetic.  Both the HIP path and the CPU
oracle consume exactly the arrays it returns, so it is the one piece of code
the two sides share.

Recipe (all from ``numpy.random.Generator(PCG64(seed))``, seed 0 by default):

* draw order: per-head parameters, then masks, then Q, K, V, then Wq, Wk;
* Q, K, V ~ N(0, 1) drawn in float32; bf16 workloads round them to bfloat16
  (round to nearest, ties to even) and keep the rounded values as the
  canonical inputs, stored here as float32 arrays holding bf16-exact values;
* block masks are uint8 ``[B, H, nQ, nK]``; rows are Q-blocks and columns
  KV-blocks (the db-SP post, scenario 2: a Q-block's work is its mask row sum);
* "diagonal forced on" sets ``mask[b, h, i, i] = 1`` after sampling.

Workloads (sizes as named by the db-SP / video-DiT / long-context settings):

1. ``tiny``     fp32, B1 H2 S256 d64, block 64, 4x4 Bernoulli(0.5) mask.
2. ``video``    bf16, B1 H24 S4096 (16 frames x 256 tokens) d64, block 64;
   heads 0-11 frame-local band (|frame(i) - frame(j)| <= 1, 4 blocks per
   frame), heads 12-23 Bernoulli(p_h), p_h ~ U[0.1, 0.5].
3. ``causal``   bf16, B1 H16 S16384 d128, block 128, lower-triangular block mask.
4. ``skewed``   bf16, B1 H40 S32768 (32 frames x 1024) d128, block 128,
   density rho_h ~ U[0.05, 0.6] with a Zipf(1.2) rank profile over rows.
5. ``topk``     bf16, B1 H16 n32768 d128, rank-32 indexer weights
   Wq, Wk ~ N(0, 1/32) of shape [128, 32] shared by all heads, top-k 512, causal.
"""
from __future__ import annotations

import dataclasses
import math
from typing import Optional

import numpy as np

__all__ = ["Workload", "make", "make_custom", "round_bf16", "CONFIG_NAMES"]

CONFIG_NAMES = {1: "tiny", 2: "video", 3: "causal", 4: "skewed", 5: "topk"}


def round_bf16(x: np.ndarray) -> np.ndarray:
    """Round float32 values to the nearest bfloat16 (ties to even), returned as float32."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32)
    bias = ((u >> np.uint32(16)) & np.uint32(1)) + np.uint32(0x7FFF)
    r = (u + bias) & np.uint32(0xFFFF0000)
    return r.view(np.float32)


@dataclasses.dataclass
class Workload:
    name: str
    B: int
    H: int
    S: int
    D: int
    dtype: str  # "f32" or "bf16"
    q: np.ndarray  # [B, H, S, D] float32 (bf16-exact when dtype == "bf16")
    k: np.ndarray
    v: np.ndarray
    block: int = 0
    n_chunks: int = 1
    layout: str = "contiguous"  # or "striped"
    mask: Optional[np.ndarray] = None  # uint8 [B, H, nQ, nK]
    wq: Optional[np.ndarray] = None  # [D, rank]
    wk: Optional[np.ndarray] = None
    rank: int = 0
    top_k: int = 0
    causal: bool = False

    @property
    def nQ(self) -> int:
        return -(-self.S // self.block) if self.block else 0

    @property
    def kind(self) -> str:
        return "topk" if self.mask is None else "block"


def _normal(rng: np.random.Generator, shape, dtype: str) -> np.ndarray:
    x = rng.standard_normal(size=shape, dtype=np.float32)
    return round_bf16(x) if dtype == "bf16" else x


def _qkv(rng, B, H, S, D, dtype, with_data=True):
    if not with_data:
        z = np.zeros((B, H, 0, D), np.float32)
        return z, z, z
    q = _normal(rng, (B, H, S, D), dtype)
    k = _normal(rng, (B, H, S, D), dtype)
    v = _normal(rng, (B, H, S, D), dtype)
    return q, k, v


def _force_diag(mask: np.ndarray) -> np.ndarray:
    n = min(mask.shape[-1], mask.shape[-2])
    idx = np.arange(n)
    mask[..., idx, idx] = 1
    return mask


def _zipf_row_counts(rng: np.random.Generator, n: int, total: int, expo: float = 1.2) -> np.ndarray:
    """Integer per-row live counts with a Zipf(expo) rank profile summing to ``total``.

    Row r gets weight pi(r)^-expo for a random rank permutation pi of 1..n, so heavy
    rows are scattered.  Counts are min(n, max(1, lam * w_r)) with lam found by
    bisection, then rounded by largest remainder (ties to the lower row index).
    """
    ranks = rng.permutation(n) + 1
    w = ranks.astype(np.float64) ** (-expo)

    def filled(lam):
        return np.minimum(float(n), np.maximum(1.0, lam * w))

    lo, hi = 0.0, float(n) / w.min() + 1.0
    for _ in range(200):
        mid = 0.5 * (lo + hi)
        if filled(mid).sum() < total:
            lo = mid
        else:
            hi = mid
    real = filled(hi)
    base = np.floor(real).astype(np.int64)
    base = np.clip(base, 1, n)
    deficit = int(total - base.sum())
    if deficit > 0:
        frac = real - np.floor(real)
        frac[base >= n] = -1.0
        order = np.lexsort((np.arange(n), -frac))
        base[order[:deficit]] += 1
    elif deficit < 0:
        frac = real - np.floor(real)
        frac[base <= 1] = 2.0
        order = np.lexsort((np.arange(n), frac))
        base[order[:-deficit]] -= 1
    assert base.sum() == total and base.min() >= 1 and base.max() <= n
    return base


def _skewed_masks(rng, B, H, n) -> np.ndarray:
    rho = rng.uniform(0.05, 0.6, size=(B, H))
    mask = np.zeros((B, H, n, n), dtype=np.uint8)
    for b in range(B):
        for h in range(H):
            total = int(round(rho[b, h] * n * n))
            counts = _zipf_row_counts(rng, n, total)
            for r in range(n):
                mask[b, h, r, r] = 1
                extra = int(counts[r]) - 1
                if extra > 0:
                    pick = rng.choice(n - 1, size=extra, replace=False)
                    cols = pick + (pick >= r)  # skip the diagonal column
                    mask[b, h, r, cols] = 1
    return mask


def make(cfg: int, seed: int = 0, layout: str = "contiguous", with_data: bool = True) -> Workload:
    """Build workload ``cfg`` (1..5) at its full size.

    ``with_data=False`` skips Q, K, V (and Wq, Wk) and returns zero-size arrays in
    their place; masks are drawn before the data, so they are unchanged.
    """
    rng = np.random.Generator(np.random.PCG64(seed))
    if cfg == 1:
        B, H, S, D, blk = 1, 2, 256, 64, 64
        n = S // blk
        mask = _force_diag((rng.random((B, H, n, n)) < 0.5).astype(np.uint8))
        q, k, v = _qkv(rng, B, H, S, D, "f32", with_data)
        return Workload("tiny", B, H, S, D, "f32", q, k, v, block=blk, n_chunks=2, mask=mask)
    if cfg == 2:
        B, H, S, D, blk = 1, 24, 4096, 64, 64
        n = S // blk
        p = rng.uniform(0.1, 0.5, size=12)
        mask = np.zeros((B, H, n, n), dtype=np.uint8)
        frame = np.arange(n) // 4
        band = (np.abs(frame[:, None] - frame[None, :]) <= 1).astype(np.uint8)
        for h in range(12):
            mask[0, h] = band
        for t in range(12):
            mask[0, 12 + t] = (rng.random((n, n)) < p[t]).astype(np.uint8)
        mask = _force_diag(mask)
        q, k, v = _qkv(rng, B, H, S, D, "bf16", with_data)
        return Workload("video", B, H, S, D, "bf16", q, k, v, block=blk, n_chunks=4, mask=mask)
    if cfg == 3:
        B, H, S, D, blk = 1, 16, 16384, 128, 128
        n = S // blk
        mask = np.broadcast_to(np.tril(np.ones((n, n), dtype=np.uint8)), (B, H, n, n)).copy()
        q, k, v = _qkv(rng, B, H, S, D, "bf16", with_data)
        return Workload("causal", B, H, S, D, "bf16", q, k, v, block=blk, n_chunks=4, layout=layout,
                        mask=mask)
    if cfg == 4:
        B, H, S, D, blk = 1, 40, 32768, 128, 128
        n = S // blk
        mask = _skewed_masks(rng, B, H, n)
        q, k, v = _qkv(rng, B, H, S, D, "bf16", with_data)
        return Workload("skewed", B, H, S, D, "bf16", q, k, v, block=blk, n_chunks=8, mask=mask)
    if cfg == 5:
        B, H, S, D, rank = 1, 16, 32768, 128, 32
        q, k, v = _qkv(rng, B, H, S, D, "bf16", with_data)
        wq = round_bf16(rng.standard_normal((D, rank), dtype=np.float32) * np.float32(math.sqrt(1.0 / rank)))
        wk = round_bf16(rng.standard_normal((D, rank), dtype=np.float32) * np.float32(math.sqrt(1.0 / rank)))
        return Workload("topk", B, H, S, D, "bf16", q, k, v, wq=wq, wk=wk, rank=rank, top_k=512,
                        causal=True)
    raise ValueError(f"unknown workload {cfg}")


def make_custom(B: int, H: int, S: int, D: int, block: int = 0, n_chunks: int = 1,
                dtype: str = "bf16", pattern: str = "bernoulli", density: float = 0.5,
                seed: int = 0, layout: str = "contiguous", top_k: int = 0, rank: int = 32,
                causal: bool = True, diag: bool = True, mask_only: bool = False) -> Workload:
    """Smaller workloads of the same families (for parity cases and edge cases).

    ``pattern``: "bernoulli" (per-entry live with probability ``density``), "causal"
    (lower-triangular), "ones", "empty" (no live tile at all), "zipf" (the skewed
    rank-profile recipe with density ``density``), or "topk" (no block mask; a rank
    ``rank`` indexer with ``top_k`` keys per query).  ``mask_only`` skips Q, K and V
    (left None) for cases that need only the mask; the mask is drawn first either way.
    """
    rng = np.random.Generator(np.random.PCG64(seed))
    if pattern == "topk":
        q, k, v = _qkv(rng, B, H, S, D, dtype)
        scale = np.float32(math.sqrt(1.0 / rank))
        wq = rng.standard_normal((D, rank), dtype=np.float32) * scale
        wk = rng.standard_normal((D, rank), dtype=np.float32) * scale
        if dtype == "bf16":
            wq, wk = round_bf16(wq), round_bf16(wk)
        return Workload(f"topk-custom-{seed}", B, H, S, D, dtype, q, k, v, wq=wq, wk=wk, rank=rank,
                        top_k=top_k, causal=causal)
    n = -(-S // block)
    if pattern == "bernoulli":
        mask = (rng.random((B, H, n, n)) < density).astype(np.uint8)
    elif pattern == "causal":
        mask = np.broadcast_to(np.tril(np.ones((n, n), dtype=np.uint8)), (B, H, n, n)).copy()
    elif pattern == "ones":
        mask = np.ones((B, H, n, n), dtype=np.uint8)
    elif pattern == "empty":
        mask = np.zeros((B, H, n, n), dtype=np.uint8)
    elif pattern == "zipf":
        rho = rng.uniform(max(1.0 / n, density * 0.5), min(1.0, density * 1.5), size=(B, H))
        mask = np.zeros((B, H, n, n), dtype=np.uint8)
        for b in range(B):
            for h in range(H):
                counts = _zipf_row_counts(rng, n, max(n, int(round(rho[b, h] * n * n))))
                for r in range(n):
                    mask[b, h, r, r] = 1
                    extra = int(counts[r]) - 1
                    if extra > 0:
                        pick = rng.choice(n - 1, size=extra, replace=False)
                        mask[b, h, r, pick + (pick >= r)] = 1
    else:
        raise ValueError(pattern)
    if diag and pattern in ("bernoulli",):
        mask = _force_diag(mask)
    q, k, v = (None, None, None) if mask_only else _qkv(rng, B, H, S, D, dtype)
    return Workload(f"{pattern}-custom-{seed}", B, H, S, D, dtype, q, k, v, block=block,
                    n_chunks=n_chunks, layout=layout, mask=mask)
