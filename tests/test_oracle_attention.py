"""Pins of oracle.attention against library routines, brute force and invariants.

Independent references used here:
* torch.nn.functional.scaled_dot_product_attention on the CPU in float64 (a library
  routine; with an all-ones block mask the masked attention must equal plain dense
  attention, and with any mask it must equal SDPA under the token mask expanded from
  the tiles);
* a pure-Python triple loop with math.exp on tiny inputs.
"""
import math

import numpy as np
import pytest
import torch

from oracle import attention as A
from sparse_mask_load_amd import workloads as W


def _sdpa(q, k, v, token_mask=None, is_causal=False):
    t = lambda x: torch.from_numpy(np.asarray(x, np.float64))
    m = None if token_mask is None else torch.from_numpy(token_mask)
    return torch.nn.functional.scaled_dot_product_attention(
        t(q), t(k), t(v), attn_mask=m, is_causal=is_causal).numpy()


def _token_mask(mask_bh, block, S):
    return np.repeat(np.repeat(mask_bh != 0, block, axis=0), block, axis=1)[:S, :S]


def test_all_ones_mask_is_dense_attention():
    w = W.make_custom(1, 3, 192, 64, block=64, pattern="ones", dtype="f32", seed=5)
    O, lse = A.masked_attention(w.q, w.k, w.v, w.mask, w.block)
    ref = _sdpa(w.q, w.k, w.v)
    assert np.abs(O - ref).max() < 1e-12
    # lse against logsumexp computed directly
    s = np.einsum("bhid,bhjd->bhij", w.q.astype(np.float64), w.k.astype(np.float64)) / 8.0
    mx = s.max(-1)
    assert np.abs(lse - (mx + np.log(np.exp(s - mx[..., None]).sum(-1)))).max() < 1e-12


@pytest.mark.parametrize("pattern,S,block", [("bernoulli", 256, 64), ("causal", 256, 32),
                                             ("bernoulli", 200, 64)])
def test_masked_attention_equals_sdpa_with_expanded_mask(pattern, S, block):
    w = W.make_custom(2, 2, S, 32, block=block, pattern=pattern, density=0.4, dtype="f32", seed=11)
    O, _ = A.masked_attention(w.q, w.k, w.v, w.mask, w.block)
    for b in range(2):
        for h in range(2):
            tm = _token_mask(w.mask[b, h], block, S)
            ref = _sdpa(w.q[b, h], w.k[b, h], w.v[b, h], token_mask=tm)
            assert np.abs(O[b, h] - ref).max() < 1e-12


def test_block_causal_equals_token_causal_on_block_diagonal_granularity():
    # block size 1 turns the block-causal mask into the ordinary token causal mask
    w = W.make_custom(1, 2, 48, 16, block=1, pattern="causal", dtype="f32", seed=2)
    O, _ = A.masked_attention(w.q, w.k, w.v, w.mask, 1)
    ref = _sdpa(w.q, w.k, w.v, is_causal=True)
    assert np.abs(O - ref).max() < 1e-12


def test_pure_python_loops_tiny():
    w = W.make_custom(1, 2, 24, 4, block=8, pattern="bernoulli", density=0.5, dtype="f32", seed=9)
    O, lse = A.masked_attention(w.q, w.k, w.v, w.mask, w.block)
    scale = 1.0 / math.sqrt(4)
    for h in range(2):
        for i in range(24):
            live = [j for j in range(24) if w.mask[0, h, i // 8, j // 8]]
            s = [scale * sum(float(w.q[0, h, i, d]) * float(w.k[0, h, j, d]) for d in range(4))
                 for j in live]
            m = max(s)
            e = [math.exp(x - m) for x in s]
            tot = sum(e)
            for d in range(4):
                ref = sum(e[n] * float(w.v[0, h, j, d]) for n, j in enumerate(live)) / tot
                assert abs(O[0, h, i, d] - ref) < 1e-12
            assert abs(lse[0, h, i] - (m + math.log(tot))) < 1e-12


def test_empty_rows_give_zero_output():
    w = W.make_custom(1, 1, 128, 16, block=32, pattern="empty", dtype="f32")
    O, lse = A.masked_attention(w.q, w.k, w.v, w.mask, 32)
    assert (O == 0).all() and np.isneginf(lse).all()


def test_mask_sensitivity():
    w = W.make_custom(1, 1, 256, 32, block=64, pattern="ones", dtype="bf16", seed=4)
    O, _ = A.masked_attention(w.q, w.k, w.v, w.mask, 64)
    m2 = w.mask.copy()
    m2[0, 0, 2, 1] = 0
    O2, _ = A.masked_attention(w.q, w.k, w.v, m2, 64)
    assert np.abs(O2[0, 0, 128:192] - O[0, 0, 128:192]).max() > 2e-2
    assert np.abs(O2[0, 0, :128] - O[0, 0, :128]).max() == 0


def test_row_sampling_matches_full():
    w = W.make_custom(1, 2, 320, 32, block=64, pattern="bernoulli", density=0.3, dtype="f32", seed=1)
    O, lse = A.masked_attention(w.q, w.k, w.v, w.mask, 64)
    rows = [(0, 0, 0), (0, 1, 319), (0, 1, 130), (0, 0, 64)]
    Os, ls = A.masked_attention(w.q, w.k, w.v, w.mask, 64, rows=rows)
    for n, (b, h, i) in enumerate(rows):
        assert np.abs(Os[n] - O[b, h, i]).max() < 1e-13 and abs(ls[n] - lse[b, h, i]) < 1e-12


@pytest.mark.parametrize("C", [1, 2, 4, 8])
@pytest.mark.parametrize("layout", ["contiguous", "striped"])
def test_chunked_merge_equals_unchunked(C, layout):
    S = 512
    w = W.make_custom(1, 2, S, 32, block=32, pattern="bernoulli", density=0.35, dtype="f32",
                      seed=C, layout=layout)
    ref, ref_lse = A.masked_attention(w.q, w.k, w.v, w.mask, 32)
    O, lse = A.chunked_attention(w.q, w.k, w.v, w.mask, 32, C, layout)
    assert np.abs(O - ref).max() < 1e-12
    fin = np.isfinite(ref_lse)
    assert np.abs(lse[fin] - ref_lse[fin]).max() < 1e-12


def test_causal_contiguous_chunks_have_empty_rows_and_merge_handles_them():
    w = W.make_custom(1, 1, 256, 16, block=32, pattern="causal", dtype="f32", seed=3)
    parts = [A.chunk_partial(w.q, w.k, w.v, w.mask, 32, 4, "contiguous", c) for c in range(4)]
    # query rows in the first quarter have no key in the last chunk: (0, -inf, 0)
    O3, m3, l3 = parts[3]
    assert np.isneginf(m3[0, 0, :64]).all() and (l3[0, 0, :64] == 0).all() and (O3[0, 0, :64] == 0).all()
    O, _ = A.merge(parts)
    ref, _ = A.masked_attention(w.q, w.k, w.v, w.mask, 32)
    assert np.abs(O - ref).max() < 1e-12


def test_merge_associative_and_order_free_and_identity():
    w = W.make_custom(1, 2, 256, 16, block=32, pattern="bernoulli", density=0.5, dtype="f32", seed=8)
    parts = [A.chunk_partial(w.q, w.k, w.v, w.mask, 32, 4, "contiguous", c) for c in range(4)]
    full, full_lse = A.merge(parts)
    # associativity: a normalised result with l = 1 and m = lse is itself a valid partial
    left, left_lse = A.merge(parts[:2])
    regrouped = [(left, left_lse, np.where(np.isneginf(left_lse), 0.0, 1.0))] + parts[2:]
    O2, _ = A.merge(regrouped)
    assert np.abs(O2 - full).max() < 1e-12
    O3, _ = A.merge(parts[::-1])
    assert np.abs(O3 - full).max() < 1e-12
    empty = (np.zeros_like(parts[0][0]), np.full_like(parts[0][1], -np.inf), np.zeros_like(parts[0][2]))
    O4, lse4 = A.merge(parts + [empty])
    assert np.abs(O4 - full).max() == 0 and np.array_equal(lse4, full_lse)
    O5, lse5 = A.merge([empty, empty])
    assert (O5 == 0).all() and np.isneginf(lse5).all()


def test_striped_equals_contiguous_result():
    w = W.make_custom(1, 2, 512, 32, block=128, pattern="causal", dtype="f32", seed=6)
    Oc, _ = A.chunked_attention(w.q, w.k, w.v, w.mask, 128, 4, "contiguous")
    Os, _ = A.chunked_attention(w.q, w.k, w.v, w.mask, 128, 4, "striped")
    assert np.abs(Oc - Os).max() < 1e-12


def test_chunk_token_sets_partition_the_sequence():
    for layout in ("contiguous", "striped"):
        toks = np.concatenate([A.chunk_token_ids(1024, 128, 4, layout, c) for c in range(4)])
        assert sorted(toks.tolist()) == list(range(1024))
    assert A.chunk_token_ids(1024, 128, 4, "striped", 1)[:3].tolist() == [1, 5, 9]
    assert A.chunk_token_ids(1024, 128, 4, "contiguous", 1)[[0, -1]].tolist() == [256, 511]


# ---- token-level causality inside live tiles ----

@pytest.mark.parametrize("pattern,S,block", [("ones", 192, 64), ("causal", 200, 64), ("causal", 256, 32)])
def test_token_causal_is_sdpa_causal(pattern, S, block):
    # an all-ones or block-lower-triangular mask contains every (i, j <= i) pair, so the
    # token-causal result is plain causal attention
    w = W.make_custom(1, 2, S, 32, block=block, pattern=pattern, dtype="f32", seed=21)
    O, lse = A.masked_attention(w.q, w.k, w.v, w.mask, block, token_causal=True)
    ref = _sdpa(w.q, w.k, w.v, is_causal=True)
    assert np.abs(O - ref).max() < 1e-12
    # the first query sees key 0 only: O = v_0 and lse = its single score
    assert np.abs(O[0, :, 0] - w.v[0, :, 0]).max() < 1e-12
    s00 = np.einsum("hd,hd->h", w.q[0, :, 0].astype(np.float64), w.k[0, :, 0].astype(np.float64)) / math.sqrt(32)
    assert np.abs(lse[0, :, 0] - s00).max() < 1e-12


def test_token_causal_bernoulli_equals_sdpa_with_combined_mask():
    S, block = 256, 32
    w = W.make_custom(2, 2, S, 16, block=block, pattern="bernoulli", density=0.4, dtype="f32", seed=22)
    w.mask[0, 0, 0] = 0
    w.mask[0, 0, 0, 3] = 1  # the first Q-block sees only a later KV block
    O, lse = A.masked_attention(w.q, w.k, w.v, w.mask, block, token_causal=True)
    tril = np.tril(np.ones((S, S), dtype=bool))
    n_empty = 0
    for b in range(2):
        for h in range(2):
            tm = _token_mask(w.mask[b, h], block, S) & tril
            has = tm.any(axis=1)
            n_empty += int((~has).sum())
            ref = _sdpa(w.q[b, h], w.k[b, h], w.v[b, h], token_mask=tm)
            assert np.abs(O[b, h][has] - ref[has]).max() < 1e-12
            # rows whose live tiles hold only later keys have no key at all
            assert (O[b, h][~has] == 0).all() and np.isneginf(lse[b, h][~has]).all()
    assert n_empty > 0  # the case is exercised


def test_token_causal_pure_python_loops_tiny():
    w = W.make_custom(1, 1, 20, 4, block=8, pattern="bernoulli", density=0.6, dtype="f32", seed=23)
    O, lse = A.masked_attention(w.q, w.k, w.v, w.mask, w.block, token_causal=True)
    for i in range(20):
        live = [j for j in range(i + 1) if w.mask[0, 0, i // 8, j // 8]]
        if not live:
            assert (O[0, 0, i] == 0).all() and lse[0, 0, i] == -np.inf
            continue
        s = [0.5 * sum(float(w.q[0, 0, i, d]) * float(w.k[0, 0, j, d]) for d in range(4)) for j in live]
        m = max(s)
        e = [math.exp(x - m) for x in s]
        for d in range(4):
            ref = sum(e[n] * float(w.v[0, 0, j, d]) for n, j in enumerate(live)) / sum(e)
            assert abs(O[0, 0, i, d] - ref) < 1e-12


@pytest.mark.parametrize("C,layout", [(4, "contiguous"), (2, "striped"), (4, "striped")])
def test_token_causal_chunked_merge_equals_unchunked(C, layout):
    S = 512
    w = W.make_custom(1, 2, S, 32, block=64, pattern="bernoulli", density=0.5, dtype="f32",
                      seed=24 + C, layout=layout)
    ref, ref_lse = A.masked_attention(w.q, w.k, w.v, w.mask, 64, token_causal=True)
    parts = [A.chunk_partial(w.q, w.k, w.v, w.mask, 64, C, layout, c, token_causal=True) for c in range(C)]
    O, lse = A.merge(parts)
    assert np.abs(O - ref).max() < 1e-12
    fin = np.isfinite(ref_lse)
    assert np.array_equal(fin, np.isfinite(lse)) and np.abs(lse[fin] - ref_lse[fin]).max() < 1e-12
    if layout == "striped":
        # query 0 has no key in chunks 1.. (their first token is c > 0)
        for c in range(1, C):
            assert np.isneginf(parts[c][1][0, :, 0]).all() and (parts[c][2][0, :, 0] == 0).all()


def test_token_causal_row_sampling_matches_full():
    w = W.make_custom(1, 2, 320, 32, block=64, pattern="bernoulli", density=0.5, dtype="f32", seed=25)
    O, lse = A.masked_attention(w.q, w.k, w.v, w.mask, 64, token_causal=True)
    rows = [(0, 0, 0), (0, 1, 319), (0, 1, 130), (0, 0, 64), (0, 0, 63)]
    Os, ls = A.masked_attention(w.q, w.k, w.v, w.mask, 64, rows=rows, token_causal=True)
    for n, (b, h, i) in enumerate(rows):
        assert np.abs(Os[n] - O[b, h, i]).max() < 1e-13
        assert (np.isneginf(ls[n]) and np.isneginf(lse[b, h, i])) or abs(ls[n] - lse[b, h, i]) < 1e-12


def test_merge_of_random_uneven_key_splits_equals_unchunked():
    """Split the KV blocks into random groups of uneven sizes (not the chunk layouts), take each
    group's normalised result as a partial (O, m = lse, l = 1; empty rows (0, -inf, 0)), and fold
    them in a random order: the merge must give the unsplit result."""
    rng = np.random.default_rng(31)
    w = W.make_custom(1, 2, 320, 16, block=32, pattern="bernoulli", density=0.5, dtype="f32", seed=31)
    ref, ref_lse = A.masked_attention(w.q, w.k, w.v, w.mask, 32)
    nK = w.mask.shape[-1]
    for trial in range(5):
        cuts = np.sort(rng.choice(np.arange(1, nK), size=rng.integers(1, 5), replace=False))
        groups = np.split(rng.permutation(nK), cuts)
        parts = []
        for g in groups:
            m_g = np.zeros_like(w.mask)
            m_g[..., g] = w.mask[..., g]
            O_g, lse_g = A.masked_attention(w.q, w.k, w.v, m_g, 32)
            parts.append((O_g, lse_g, np.where(np.isneginf(lse_g), 0.0, 1.0)))
        order = rng.permutation(len(parts))
        O, lse = A.merge([parts[i] for i in order])
        assert np.abs(O - ref).max() < 1e-12
        fin = np.isfinite(ref_lse)
        assert np.array_equal(fin, np.isfinite(lse)) and np.abs(lse[fin] - ref_lse[fin]).max() < 1e-12


@pytest.mark.parametrize("layout,token_causal,scale", [("contiguous", False, None), ("striped", False, 1.0),
                                                        ("contiguous", True, 0.7), ("striped", True, None)])
def test_chunk_partial_each_of_o_m_l_pure_python_loops(layout, token_causal, scale):
    """Each of a chunk partial's O, m and l on its own, by a pure-Python loop over the chunk's
    live keys: m is the row maximum over the keys of that chunk only (not over the Q-block or
    the whole row), l = sum exp(s - m) and O = sum exp(s - m) v, unnormalised."""
    S, D, blk, C = 32, 4, 8, 2
    w = W.make_custom(1, 2, S, D, block=blk, pattern="bernoulli", density=0.6, dtype="f32", seed=17,
                      layout=layout)
    sc = 1.0 / math.sqrt(D) if scale is None else scale
    for c in range(C):
        O, M, L = A.chunk_partial(w.q, w.k, w.v, w.mask, blk, C, layout, c, scale=scale,
                                  token_causal=token_causal)
        rows = [(0, h, i) for h in range(2) for i in range(S)]
        Or, Mr, Lr = A.chunk_partial(w.q, w.k, w.v, w.mask, blk, C, layout, c, scale=scale,
                                     token_causal=token_causal, rows=rows)
        for n, (_, h, i) in enumerate(rows):
            if layout == "contiguous":
                keys = range(c * (S // C), (c + 1) * (S // C))
            else:
                keys = range(c, S, C)
            keys = [j for j in keys if w.mask[0, h, i // blk, j // blk] and not (token_causal and j > i)]
            if not keys:
                assert M[0, h, i] == -math.inf and L[0, h, i] == 0 and (O[0, h, i] == 0).all()
                assert Mr[n] == -math.inf and Lr[n] == 0 and (Or[n] == 0).all()
                continue
            s = [sc * sum(float(w.q[0, h, i, d]) * float(w.k[0, h, j, d]) for d in range(D)) for j in keys]
            m = max(s)
            e = [math.exp(x - m) for x in s]
            for got_m, got_l, got_o in ((M[0, h, i], L[0, h, i], O[0, h, i]), (Mr[n], Lr[n], Or[n])):
                assert abs(got_m - m) < 1e-12
                assert abs(got_l - sum(e)) < 1e-12
                for d in range(D):
                    assert abs(got_o[d] - sum(e[t] * float(w.v[0, h, j, d]) for t, j in enumerate(keys))) < 1e-12


def test_merge_equals_sequential_online_softmax_fold():
    """The merge's closed form equals the 6D notes' one-part-at-a-time update (section 2.1,
    with the lost multiplications restored), run here as a pure-Python loop, including empty
    parts at the start, in the middle and at the end."""
    rng = np.random.default_rng(23)
    n_parts, rows, D = 5, 7, 3
    O = rng.standard_normal((n_parts, rows, D))
    m = rng.standard_normal((n_parts, rows)) * 3
    l = rng.uniform(0.5, 4, (n_parts, rows))
    for p, r in ((0, 1), (2, 1), (4, 1), (0, 2), (1, 2), (2, 2), (3, 2), (4, 2), (4, 5)):
        O[p, r], m[p, r], l[p, r] = 0.0, -math.inf, 0.0
    got, got_lse = A.merge([(O[p], m[p], l[p]) for p in range(n_parts)])
    for r in range(rows):
        acc_o, acc_m, acc_l = [0.0] * D, -math.inf, 0.0
        for p in range(n_parts):
            new_m = max(acc_m, m[p, r])
            if new_m == -math.inf:
                continue  # both sides hold nothing yet
            a, b = math.exp(acc_m - new_m), math.exp(m[p, r] - new_m)
            acc_l = a * acc_l + b * l[p, r]
            acc_o = [a * acc_o[d] + b * O[p, r, d] for d in range(D)]
            acc_m = new_m
        if acc_l == 0:
            assert (got[r] == 0).all() and got_lse[r] == -math.inf
            continue
        for d in range(D):
            assert abs(got[r, d] - acc_o[d] / acc_l) < 1e-12
        assert abs(got_lse[r] - (acc_m + math.log(acc_l))) < 1e-12
