"""The allocation-free entry point (sparse_attn_fwd_noalloc) against the entry points it stands
for: a plan made with the device order followed by sparse_attn_fwd.  Both run the same kernels on
the same work list, so outputs must agree bit for bit; two calls in a row, the second on a
smaller problem, check that the second call is not affected by what the first left in the
library's work array.  Each output is also checked against the oracle on sampled rows."""
import numpy as np
import pytest
import torch

from oracle import attention as A
from sparse_mask_load_amd import binding as bd
from sparse_mask_load_amd import workloads as W
from tests import gpu_util as G

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    bd.lib()  # fails loudly if the library is missing


def _check(w, seed, q_pairs=False):
    print(f"noalloc case: B{w.B} H{w.H} S{w.S} d{w.D} block {w.block} C{w.n_chunks} {w.layout} pairs {q_pairs}",
          flush=True)
    q, k, v = G.upload(w)
    C = w.n_chunks
    prob = bd.make_problem(q, w.block, C, w.layout, q_pairs=q_pairs)
    mask = torch.from_numpy(np.ascontiguousarray(w.mask)).cuda()
    plan = bd.sparse_attn_plan(prob, "block", mask=mask, order="lpt_device")
    # full mode over every chunk
    o_ref = G.empty_like_qkv(q)
    bd.sparse_attn_fwd(plan, q, k, v, 0, C, o=o_ref)
    o_na = G.empty_like_qkv(q)
    bd.sparse_attn_fwd_noalloc(prob, mask, q, k, v, 0, C, o=o_na)
    torch.cuda.synchronize()
    assert torch.equal(o_na, o_ref)
    rows = G.sample_rows(w, 48, seed=seed)
    idx = tuple(np.array(rows).T)
    ref, _ = A.masked_attention(w.q, w.k, w.v, w.mask, w.block, rows=rows)
    G.assert_close(G.to64(o_na)[idx], ref, G.tol_for(w), "noalloc full")
    # partial mode: every chunk in one call, and the last chunk alone (its own list)
    B, H, S, D = q.shape
    for c0, c1 in ((0, C), (C - 1, C)):
        n = c1 - c0
        parts = [torch.empty((n, B, H, S, D), dtype=torch.float32, device="cuda") for _ in range(2)]
        ms = [torch.empty((n, B, H, S), dtype=torch.float32, device="cuda") for _ in range(2)]
        ls = [torch.empty((n, B, H, S), dtype=torch.float32, device="cuda") for _ in range(2)]
        bd.sparse_attn_fwd(plan, q, k, v, c0, c1, o_part=parts[0], m_part=ms[0], l_part=ls[0])
        bd.sparse_attn_fwd_noalloc(prob, mask, q, k, v, c0, c1, o_part=parts[1], m_part=ms[1], l_part=ls[1])
        torch.cuda.synchronize()
        assert torch.equal(parts[1], parts[0]) and torch.equal(ms[1], ms[0]) and torch.equal(ls[1], ls[0])
    plan.close()


def test_noalloc_matches_plan_and_forward_on_two_calls():
    # the causal workload at full size, then a smaller ragged problem in fewer bins' worth of items
    _check(W.make(3), seed=1)
    _check(W.make_custom(1, 3, 1000, 64, block=128, n_chunks=2, dtype="bf16", pattern="bernoulli", density=0.5,
                         seed=41), seed=2)


def test_noalloc_with_q_block_pairs_on_two_calls():
    # pair items: the causal workload, then an odd number of Q-blocks (a lone last pair row),
    # then striped chunks
    _check(W.make(3), seed=3, q_pairs=True)
    _check(W.make_custom(1, 3, 1152, 128, block=128, n_chunks=3, dtype="bf16", pattern="bernoulli", density=0.5,
                         seed=42), seed=4, q_pairs=True)
    _check(W.make_custom(1, 2, 2048, 128, block=128, n_chunks=4, dtype="bf16", pattern="causal", seed=43,
                         layout="striped"), seed=5, q_pairs=True)


def test_noalloc_rejects_oversized_problems_on_the_gpu():
    w = W.make_custom(1, 1, 256, 64, block=64, n_chunks=2, dtype="bf16", pattern="ones")
    q, k, v = G.upload(w)
    prob = bd.make_problem(q, w.block, w.n_chunks, w.layout)
    mask = torch.from_numpy(np.ascontiguousarray(w.mask)).cuda()
    with pytest.raises(bd.SparseAttnError) as e:
        bd.sparse_attn_fwd_noalloc(prob, mask, q, k, v, 0, 2, o=G.empty_like_qkv(q), num_bins=2048)
    assert e.value.status == bd.SA_ERR_UNSUPPORTED
