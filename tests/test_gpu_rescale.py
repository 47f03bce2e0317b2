"""GPU parity on inputs that drive the bf16 kernel's online-softmax rescale.

The kernel rescales a row's O and l by exp(m_old - m_new) (6D notes, section 2.1, the alpha
factor of the update) only when the row maximum grows by more than 8 log2 units within a
chunk; ``tests/test_rescale_inputs.py`` shows on the CPU that each case here does so many
times in both modes.  Every row of the full-mode output, every chunk partial (m, l and O / l)
and the merged output with its lse are compared with the oracle at the case's softmax scale.
"""
import numpy as np
import pytest
import torch

from oracle import attention as A
from sparse_mask_load_amd import binding as bd
from tests import gpu_util as G
from tests import lazy_rescale as LR

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    bd.lib()  # fails loudly if the library is missing


@pytest.mark.parametrize("n", range(len(LR.RESCALE_CASES)), ids=[LR.rescale_case_id(c) for c in LR.RESCALE_CASES])
def test_rescale_every_row(n):
    w, scale, tc = LR.make_rescale_case(n)
    print(f"rescale case {n}: {LR.rescale_case_id(LR.RESCALE_CASES[n])}", flush=True)
    q, k, v = G.upload(w)
    prob = bd.make_problem(q, w.block, w.n_chunks, w.layout, scale=scale or 0.0, token_causal=tc)
    mask = torch.from_numpy(np.ascontiguousarray(w.mask)).cuda()
    plan = bd.sparse_attn_plan(prob, "block", mask=mask)
    C = w.n_chunks
    ref, ref_lse = A.masked_attention(w.q, w.k, w.v, w.mask, w.block, scale=scale, token_causal=tc)
    o = G.run_full(plan, q, k, v)
    G.assert_close(G.to64(o), ref, G.BF16_TOL, "full")
    op, mp, lp = G.run_partial(plan, q, k, v, 0, C)
    for c in range(C):
        Oc, Mc, Lc = A.chunk_partial(w.q, w.k, w.v, w.mask, w.block, C, w.layout, c, scale=scale,
                                     token_causal=tc)
        got_m = G.to64(mp[c])
        assert np.array_equal(np.isneginf(got_m), np.isneginf(Mc)), "empty-chunk rows differ"
        fin = np.isfinite(Mc)
        if fin.any():
            G.assert_close(got_m[fin], Mc[fin], (2e-3, 1e-4), f"m chunk {c}")
            G.assert_close(G.to64(lp[c])[fin] / Lc[fin], np.ones(fin.sum()), G.ROWSUM_TOL, f"l chunk {c}")
            on = G.to64(op[c])[fin] / G.to64(lp[c])[fin][:, None]
            G.assert_close(on, Oc[fin] / Lc[fin][:, None], G.BF16_TOL, f"O/l chunk {c}")
        assert (G.to64(op[c])[~fin] == 0).all() and (G.to64(lp[c])[~fin] == 0).all()
    om, lse = G.merge(op, mp, lp)
    G.assert_close(G.to64(om), ref, G.BF16_TOL, "merged")
    got_lse = G.to64(lse)
    assert np.array_equal(np.isneginf(got_lse), np.isneginf(ref_lse))
    fin = np.isfinite(ref_lse)
    G.assert_close(got_lse[fin], ref_lse[fin], G.ROWSUM_TOL, "lse")
    plan.close()
