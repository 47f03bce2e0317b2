"""Oracle: block-masked attention, per-chunk partials and the online-softmax merge.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).  fp64 numpy, no blocking
beyond processing one Q-block of rows at a time to bound memory.

Definitions followed:

* Masked attention (the result the block-sparse method must reach exactly):
  ``O[i] = sum_j softmax_j(s_ij) v_j`` with ``s_ij = scale * <q_i, k_j>`` when
  ``mask[floor(i / block), floor(j / block)]`` is non-zero and ``-inf``
  otherwise; ``scale = 1 / sqrt(d)``.  Rows are Q-blocks and columns KV-blocks
  (db-SP post, scenario 2 bullets).  A row with no live key gets O = 0 and
  lse = -inf.
* Per-chunk partial = the ring step's ``flash_attention(Q, K, V) -> (O_step,
  m_step, l_step)`` of the 6D-parallel notes, section 2.1: ``m`` is the row max
  of the live scores in the chunk, ``l = sum exp(s - m)`` and ``O`` is the
  UNNORMALISED ``sum exp(s - m) v`` (the pseudocode marks the accumulator as
  unnormalised and divides once at the end).  Rows with no live key in the
  chunk give ``(O, m, l) = (0, -inf, 0)``.
* Merge of partials over disjoint key sets (the same section's online-softmax
  update, whose multiplication signs the page lost): every partial holds its
  exponentials relative to its own maximum, so with ``M = max_p m_p`` the
  combined row is ``sum_p exp(m_p - M) O_p / sum_p exp(m_p - M) l_p`` and its
  log-sum-exp is ``M + log(sum_p exp(m_p - M) l_p)``.  The page folds the parts
  one at a time; the fold reaches exactly this closed form, which is what is
  written here.  Parts with ``m_p = -inf`` have weight 0; a row whose every
  part is empty gives O = 0 and lse = -inf (the page is silent on such rows).
* Token-level causality (option ``token_causal``): the mask above decides which
  tiles exist; inside them key j is also dropped for query i when ``j > i``
  (positions in the original sequence, also for striped chunks).  With an
  all-ones block mask this is plain causal softmax attention.  Rows left with
  no key behave as rows with no live key above.
* Chunk composition: contiguous chunk c holds KV blocks
  ``[c*nK/C, (c+1)*nK/C)``; striped chunk c holds tokens ``j`` with
  ``j mod C == c`` (section 2.3's striped attention, "token i -> chunk i mod C").
"""
from __future__ import annotations

import math
from typing import List, Optional, Sequence, Tuple

import numpy as np

NEG_INF = -np.inf


def default_scale(D: int) -> float:
    return 1.0 / math.sqrt(D)


def _f64(x) -> np.ndarray:
    return np.asarray(x, dtype=np.float64)


def chunk_token_ids(S: int, block: int, n_chunks: int, layout: str, c: int) -> np.ndarray:
    """KV token indices that form chunk ``c``."""
    if layout == "contiguous":
        nK = -(-S // block)
        per = nK // n_chunks
        lo = c * per * block
        hi = min(S, (c + 1) * per * block)
        return np.arange(lo, hi)
    if layout == "striped":
        return np.arange(c, S, n_chunks)
    raise ValueError(layout)


def _key_live(mask_row: np.ndarray, block: int, S: int) -> np.ndarray:
    """Token-level liveness of every key for one Q-block's mask row."""
    return np.repeat(mask_row != 0, block)[:S]


def _softmax_rows(s):
    """Row max, exp(s - max) and row sum of a score matrix whose rows may be all -inf.

    Such rows get m = -inf, p = 0 and l = 0.
    """
    m = s.max(axis=1)
    m_safe = np.where(np.isneginf(m), 0.0, m)
    p = np.exp(s - m_safe[:, None])  # exp(-inf) = 0
    return m, p, p.sum(axis=1)


def _drop_future(s, q_pos, k_pos):
    """Token-level causality: score (i, j) becomes -inf when key position j > query position i."""
    return np.where(k_pos[None, :] > q_pos[:, None], NEG_INF, s)


def masked_attention(q, k, v, mask, block: int, scale: Optional[float] = None,
                     rows: Optional[Sequence[Tuple[int, int, int]]] = None, token_causal: bool = False):
    """Dense softmax attention with dead (Q-block, KV-block) tiles set to -inf.

    q, k, v: [B, H, S, D]; mask: [B, H, nQ, nK].  Returns ``(O, lse)`` in fp64,
    shaped [B, H, S, D] / [B, H, S], or [len(rows), D] / [len(rows)] when ``rows``
    (a list of (b, h, token)) selects individual output rows.  ``token_causal``
    also drops keys after each query inside live tiles.
    """
    q, k, v = _f64(q), _f64(k), _f64(v)
    B, H, S, D = q.shape
    sc = default_scale(D) if scale is None else float(scale)
    if rows is not None:
        out = np.zeros((len(rows), D))
        lse = np.full(len(rows), NEG_INF)
        for n, (b, h, i) in enumerate(rows):
            live = _key_live(mask[b, h, i // block], block, S)
            if token_causal:
                live = live & (np.arange(S) <= i)
            if not live.any():
                continue
            s = sc * (k[b, h][live] @ q[b, h, i])
            m = s.max()
            p = np.exp(s - m)
            out[n] = (p @ v[b, h][live]) / p.sum()
            lse[n] = m + math.log(p.sum())
        return out, lse
    out = np.zeros((B, H, S, D))
    lse = np.full((B, H, S), NEG_INF)
    nQ = -(-S // block)
    for b in range(B):
        for h in range(H):
            for qi in range(nQ):
                r0, r1 = qi * block, min(S, (qi + 1) * block)
                live = _key_live(mask[b, h, qi], block, S)
                if not live.any():
                    continue
                s = sc * (q[b, h, r0:r1] @ k[b, h][live].T)
                if token_causal:
                    s = _drop_future(s, np.arange(r0, r1), np.nonzero(live)[0])
                m, p, l = _softmax_rows(s)
                has = l > 0
                out[b, h, r0:r1][has] = (p[has] @ v[b, h][live]) / l[has, None]
                lse[b, h, r0:r1][has] = m[has] + np.log(l[has])
    return out, lse


def chunk_partial(q, k, v, mask, block: int, n_chunks: int, layout: str, c: int,
                  scale: Optional[float] = None, token_causal: bool = False,
                  rows: Optional[Sequence[Tuple[int, int, int]]] = None):
    """One ring step's partial ``(O_unnormalised, m, l)`` over the KV tokens of chunk ``c``.

    Shapes: O [B, H, S, D], m and l [B, H, S], fp64; or [len(rows), D] and
    [len(rows)] when ``rows`` (a list of (b, h, token)) selects individual rows.
    """
    q, k, v = _f64(q), _f64(k), _f64(v)
    B, H, S, D = q.shape
    sc = default_scale(D) if scale is None else float(scale)
    toks = chunk_token_ids(S, block, n_chunks, layout, c)
    if rows is not None:
        O = np.zeros((len(rows), D))
        M = np.full(len(rows), NEG_INF)
        L = np.zeros(len(rows))
        for n, (b, h, i) in enumerate(rows):
            kt = toks[_key_live(mask[b, h, i // block], block, S)[toks]]
            if token_causal:
                kt = kt[kt <= i]
            if kt.shape[0] == 0:
                continue
            s = sc * (k[b, h, kt] @ q[b, h, i])
            M[n] = s.max()
            p = np.exp(s - M[n])
            L[n] = p.sum()
            O[n] = p @ v[b, h, kt]
        return O, M, L
    O = np.zeros((B, H, S, D))
    M = np.full((B, H, S), NEG_INF)
    L = np.zeros((B, H, S))
    nQ = -(-S // block)
    for b in range(B):
        for h in range(H):
            for qi in range(nQ):
                r0, r1 = qi * block, min(S, (qi + 1) * block)
                live = _key_live(mask[b, h, qi], block, S)[toks]
                if not live.any():
                    continue
                kt = toks[live]
                s = sc * (q[b, h, r0:r1] @ k[b, h, kt].T)
                if token_causal:
                    s = _drop_future(s, np.arange(r0, r1), kt)
                m, p, l = _softmax_rows(s)
                O[b, h, r0:r1] = p @ v[b, h, kt]
                M[b, h, r0:r1] = m
                L[b, h, r0:r1] = l
    return O, M, L


def merge(parts: List[Tuple[np.ndarray, np.ndarray, np.ndarray]]):
    """Combine per-chunk partials ``[(O, m, l), ...]`` into the normalised result.

    O: [..., D]; m, l: [...].  Returns ``(O_normalised, lse)``: each partial is
    weighted by ``exp(m_p - M)`` with ``M`` the largest of the parts' maxima; rows
    whose every partial is empty give O = 0 and lse = -inf.
    """
    m_all = np.stack([_f64(m) for _, m, _ in parts])  # [P, ...]
    M = m_all.max(axis=0)
    none = np.isneginf(M)
    M_safe = np.where(none, 0.0, M)
    weight = np.exp(m_all - M_safe)  # exp(-inf) = 0 for empty parts
    den = sum(w * _f64(l) for w, (_, _, l) in zip(weight, parts))
    num = sum(w[..., None] * _f64(O) for w, (O, _, _) in zip(weight, parts))
    pos = den > 0
    O = np.where(pos[..., None], num / np.where(pos, den, 1.0)[..., None], 0.0)
    with np.errstate(divide="ignore"):
        lse = np.where(pos, M_safe + np.log(np.where(pos, den, 1.0)), NEG_INF)
    return O, lse


def chunked_attention(q, k, v, mask, block: int, n_chunks: int, layout: str,
                      scale: Optional[float] = None, token_causal: bool = False):
    """The ring emulation on one device: every chunk's partial, then the merge."""
    parts = [chunk_partial(q, k, v, mask, block, n_chunks, layout, c, scale, token_causal)
             for c in range(n_chunks)]
    return merge(parts)
