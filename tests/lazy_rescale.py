"""Replay of the bf16 attention kernel's lazy reference maximum, on the CPU.

The kernel keeps, per query row, the exact running maximum of the scaled scores
for the exported m, but subtracts a separate reference maximum inside the
exponent.  A wave of 32 query rows holds one half of the keys of every tile
(key blocks kh*BLK/64 .. of the tile) and moves its rows' references only when
some row's maximum over the wave's keys of the current tile exceeds that row's
reference by more than 8 (log2 units).  Then every row that exceeded it takes
its running maximum as the new reference, and — unless no row of the wave had a
finite reference yet — every row's O and l are multiplied by
exp2(old reference - new reference).  That multiplication (the alpha rescale of
the online softmax) is what the tests built on this module must reach.

This module decides nothing about the result: it only counts how often the
rescale of an already non-empty row happens for a given input, so that a test
can show that its input drives the kernel through that branch.
"""
from __future__ import annotations

import math

import numpy as np

SLACK_LOG2 = 8.0


def _tile_sequence(mask_row, S, block, C, layout, c0, c1):
    """(chunk, key tokens of the tile in kernel order; -1 for dead or absent keys) per live tile."""
    nK = -(-S // block)
    per = nK // C
    out = []
    for c in range(c0, c1):
        if layout == "contiguous":
            for j in range(c * per, (c + 1) * per):
                if mask_row[j]:
                    toks = j * block + np.arange(block)
                    toks[toks >= S] = -1
                    out.append((c, toks))
        else:
            for t in range(per):
                toks = c + C * (t * block + np.arange(block))
                live = mask_row[toks // block] != 0
                if live.any():
                    toks = np.where(live, toks, -1)
                    out.append((c, toks))
    return out


def count_rescales(w, scale=None, c0=0, c1=None, full=True, token_causal=False, heads=None, pairs=False):
    """Number of (row, tile) events where the kernel rescales a row that already holds a finite
    reference, over every item of heads ``heads`` (all by default), in full mode (one state over
    the chunk range) or partial mode (the state restarts at every chunk).  ``pairs``: the
    Q-block-pair mapping, where a wave holds all keys of every tile and checks its rows after
    each 32-key block (a tile that is live only for the other Q-block of the pair adds nothing)."""
    c1 = w.n_chunks if c1 is None else c1
    blk, S = w.block, w.S
    nb = blk // 64  # 32-key blocks per wave
    sl2 = (1.0 / math.sqrt(w.D) if not scale else scale) / math.log(2.0)
    events = 0
    for b in range(w.B):
        for h in (range(w.H) if heads is None else heads):
            s = (np.asarray(w.q[b, h], np.float64) @ np.asarray(w.k[b, h], np.float64).T) * sl2
            for qb in range(-(-S // blk)):
                tiles = _tile_sequence(w.mask[b, h, qb], S, blk, w.n_chunks, w.layout, c0, c1)
                for rg in range(blk // 32):
                    rows = np.arange(qb * blk + rg * 32, min(S, qb * blk + rg * 32 + 32))
                    if rows.size == 0:
                        continue
                    for kh in range(1 if pairs else 2):
                        m_ref = np.full(rows.size, -np.inf)
                        m_true = np.full(rows.size, -np.inf)
                        cur = c0
                        steps = [(c, toks[i:i + 32]) for c, toks in tiles for i in range(0, blk, 32)] if pairs \
                            else [(c, toks[kh * nb * 32:(kh + 1) * nb * 32]) for c, toks in tiles]
                        for c, kt in steps:
                            if not full and c != cur:
                                m_ref[:] = -np.inf
                                m_true[:] = -np.inf
                                cur = c
                            sub = s[np.ix_(rows, np.maximum(kt, 0))]
                            dead = np.broadcast_to(kt < 0, sub.shape)
                            if token_causal:
                                dead = dead | (kt[None, :] > rows[:, None])
                            mx = np.where(dead, -np.inf, sub).max(axis=1)
                            m_true = np.maximum(m_true, mx)
                            moved = mx > m_ref + SLACK_LOG2
                            if not moved.any():
                                continue
                            new_ref = np.where(moved, m_true, m_ref)
                            if np.isfinite(m_ref).any():
                                events += int((np.isfinite(m_ref) & (new_ref > m_ref)).sum())
                            m_ref = new_ref
    return events


# Inputs on which the rescale happens, one per kernel variant family: (B, H, S, D, block, C,
# mask pattern, density, layout, softmax scale (None: 1/sqrt(D)), factor applied to the K rows
# of odd KV blocks, token_causal).  A scale of 1.0 spreads N(0,1) scores over about sqrt(D)
# natural-log units, and K rows amplified by 4-8 in every other block raise a row's maximum
# from one tile to the next; either drives row maxima up by more than 8 log2 units inside a
# chunk.  Powers of two keep the amplified bf16 values exact.
RESCALE_CASES = [
    (1, 2, 1024, 128, 128, 2, "causal", 0.0, "contiguous", None, 8, False),   # full tiles, d128 b128
    (1, 2, 1024, 64, 64, 4, "bernoulli", 0.6, "contiguous", 1.0, 1, False),   # full tiles, d64 b64
    (1, 2, 768, 128, 64, 2, "ones", 0.0, "contiguous", None, 4, False),       # full tiles, d128 b64
    (1, 2, 1000, 64, 128, 1, "bernoulli", 0.5, "contiguous", 1.0, 1, False),  # ragged last block
    (1, 2, 2048, 128, 128, 4, "causal", 0.0, "striped", 1.0, 1, False),       # striped
    (1, 2, 1024, 128, 128, 2, "ones", 0.0, "contiguous", None, 8, True),      # token-causal, full tiles
    (1, 2, 1024, 64, 64, 2, "ones", 0.0, "striped", 1.0, 1, True),            # token-causal, striped
    (1, 2, 1152, 128, 128, 3, "bernoulli", 0.6, "contiguous", 1.0, 1, False),  # odd nQ (a lone last pair row)
]


def rescale_case_id(c):
    return f"{c[6]}-S{c[2]}-d{c[3]}-b{c[4]}-C{c[5]}-{c[8][:4]}-sc{c[9]}-x{c[10]}{'-tc' if c[11] else ''}"


def make_rescale_case(n):
    """Workload of RESCALE_CASES[n] (seeded) with its K amplification applied."""
    from sparse_mask_load_amd import workloads as W

    B, H, S, D, blk, C, pattern, dens, layout, scale, amp, tc = RESCALE_CASES[n]
    w = W.make_custom(B, H, S, D, block=blk, n_chunks=C, pattern=pattern, density=dens, seed=300 + n,
                      layout=layout)
    if amp != 1:
        k = w.k.copy()
        for j in range(1, -(-S // blk), 2):
            k[:, :, j * blk:(j + 1) * blk] *= np.float32(amp)
        w.k = k
    return w, scale, tc
