"""Helpers for the GPU parity tests: move workloads to the device and run the C ABI."""
import math

import numpy as np
import torch

from sparse_mask_load_amd import binding as bd

BF16_TOL = (2e-2, 2e-3)  # max-abs, mean-abs (bf16 in, fp32 accumulate)
F32_TOL = (1e-4, 1e-4)
# The bf16 kernel's row sum l adds the bf16-rounded P values (the same ones that multiply V).
# Rounding to nearest changes each term p_i by a relative e_i with |e_i| <= u = 2^-9, so in
# every row |dl / l| = |sum p_i e_i| / sum p_i <= u; the fp32 sums around it add at most
# n * 2^-24 <= 2^-10 for rows of up to 16384 keys, so the max bound is 2^-9 + 2^-10 < 2^-8.
# Over many rows the mean is bounded by the root mean square: modelling the e_i as independent
# and uniform on [-u, u] (round-to-nearest errors are unbiased), E (dl / l)^2 =
# (u^2 / 3) sum p_i^2 / (sum p_i)^2 <= u^2 / 3, so E |dl / l| <= u / sqrt(3), reached when one
# key dominates the row (a peaked softmax); 2^-12 more covers the fp32 sums.  lse = m + log(l)
# has the same absolute error.
ROWSUM_TOL = (2.0 ** -8, 2.0 ** -9 / math.sqrt(3.0) + 2.0 ** -12)


def tol_for(w):
    return BF16_TOL if w.dtype == "bf16" else F32_TOL


def dev(x, dtype):
    t = torch.from_numpy(np.ascontiguousarray(x))
    return t.to(device="cuda", dtype=dtype)


def upload(w, layout_bshd=False):
    """Q, K, V on the GPU ([B, H, S, D]; optionally as permuted views of [B, S, H, D] storage)."""
    dt = torch.bfloat16 if w.dtype == "bf16" else torch.float32
    out = []
    for x in (w.q, w.k, w.v):
        if layout_bshd:
            t = dev(np.transpose(x, (0, 2, 1, 3)), dt).permute(0, 2, 1, 3)
        else:
            t = dev(x, dt)
        out.append(t)
    return out


def empty_like_qkv(q):
    """Output tensor with the same strides as q."""
    return torch.empty_strided(q.shape, q.stride(), dtype=q.dtype, device=q.device)


def plan_block(w, q, order="lpt", num_bins=0, layout=None, token_causal=False, q_pairs=False, scale=0.0):
    prob = bd.make_problem(q, w.block, w.n_chunks, layout or w.layout, scale=scale, token_causal=token_causal,
                           q_pairs=q_pairs)
    mask = torch.from_numpy(np.ascontiguousarray(w.mask)).cuda()
    plan = bd.sparse_attn_plan(prob, "block", mask=mask, num_bins=num_bins, order=order)
    del mask  # the plan keeps its own copy
    return plan


def run_full(plan, q, k, v, c0=0, c1=None, trace=None):
    o = empty_like_qkv(q)
    bd.sparse_attn_fwd(plan, q, k, v, c0, c1, o=o, trace=trace)
    torch.cuda.synchronize()
    return o


def run_partial(plan, q, k, v, c0, c1):
    B, H, S, D = q.shape
    n = c1 - c0
    o_part = torch.empty((n, B, H, S, D), dtype=torch.float32, device="cuda")
    m_part = torch.empty((n, B, H, S), dtype=torch.float32, device="cuda")
    l_part = torch.empty((n, B, H, S), dtype=torch.float32, device="cuda")
    bd.sparse_attn_fwd(plan, q, k, v, c0, c1, o_part=o_part, m_part=m_part, l_part=l_part)
    torch.cuda.synchronize()
    return o_part, m_part, l_part


def merge(o_part, m_part, l_part, out_dtype="bf16", want_lse=True):
    n, B, H, S, D = o_part.shape
    rows = B * H * S
    dt = torch.bfloat16 if out_dtype == "bf16" else torch.float32
    out = torch.empty((B, H, S, D), dtype=dt, device="cuda")
    lse = torch.empty((B, H, S), dtype=torch.float32, device="cuda") if want_lse else None
    bd.chunk_merge([o_part[i] for i in range(n)], [m_part[i] for i in range(n)], [l_part[i] for i in range(n)],
                   rows, D, out, out_dtype, lse)
    torch.cuda.synchronize()
    return out, lse


def to64(t):
    return t.detach().to(torch.float64).cpu().numpy()


def assert_close(got, ref, tol, what=""):
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    assert got.shape == ref.shape, (got.shape, ref.shape)
    assert np.isfinite(got).all(), f"{what}: non-finite output"
    err = np.abs(got - ref)
    mx, mean = float(err.max()) if err.size else 0.0, float(err.mean()) if err.size else 0.0
    assert mx <= tol[0] and mean <= tol[1], f"{what}: max-abs {mx:.3g} mean-abs {mean:.3g} (tol {tol})"
    return mx, mean


def sample_rows(w, n=96, seed=0):
    """Seeded sample of (b, h, token) rows plus the first/last rows of edge blocks and heads."""
    rng = np.random.default_rng(seed)
    n = min(n, w.B * w.H * w.S)  # there are only that many distinct rows
    rows = {(0, 0, 0), (0, w.H - 1, w.S - 1), (0, 0, w.S - 1), (0, w.H - 1, 0)}
    if w.block:
        rows |= {(0, w.H // 2, w.block - 1), (0, w.H // 2, w.block), (0, 1 % w.H, w.S - w.block)}
    while len(rows) < n:
        rows.add((int(rng.integers(0, w.B)), int(rng.integers(0, w.H)), int(rng.integers(0, w.S))))
    return sorted(rows)
