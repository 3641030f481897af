"""GPU parity of the float32 backward (float32 inputs, float32 MFMA, no rounding of P or
dS) against the float64 oracle.

The recomputation backward of the marketmaker.cc attention page (the section on the
backward pass recomputing rather than storing), on float32 inputs.

Tolerance, derived from the arithmetic (u = 2^-24): every gradient element is a sum of
products whose factors carry relative errors from float32 dot products of length d (the
scores and dP), the exponential of the score in log2 units (its absolute error, at most
u (d S_hat + |LSE|) with S_hat the largest scale * sum_c |q_c k_c|, becomes a relative
error of P) and sums of up to N terms. With A the sum of the absolute values of the terms
of an element (for dV: sum_i P_ij |dO_ic|; for dK and dQ the same with
|dS| <= P (sum_c |dO_c V_c| + sum_c |dO_c O_c|) in place of P, times scale), the bound is
    |err| <= 4 u (d S_hat + |LSE|_max + N + 16) A + 1e-7.
"""

import math

import numpy as np
import pytest
import torch

import oracle
from synth import WORKLOADS, bias_tensor, key_ranges, normal, qkv_inputs
from tests.util import assert_fwd_close, np64

pytestmark = pytest.mark.gpu

fa = pytest.importorskip("exact_io_aware_flash_amd")
DEV = "cuda:0"
U = 2.0 ** -24


def grad_bounds(q, k, v, do, scale, causal, with_ds=False, **mask):
    """Per-element bounds on |dQ|, |dK|, |dV| errors (module docstring), float64; with
    with_ds also the bound on |dS| errors [B, H, N_q, N_k] and the masked entries."""
    B, H, nq, d = q.shape
    nk = k.shape[2]
    o, lse = oracle.attention_forward(q, k, v, scale, causal=causal, **mask)
    bq, bk, bv = np.zeros(q.shape), np.zeros(k.shape), np.zeros(v.shape)
    bds, masked = np.zeros((B, H, nq, nk)), np.zeros((B, H, nq, nk), dtype=bool)
    for b in range(B):
        for h in range(H):
            p = oracle.attention_probabilities(q, k, scale, b, h, causal, **mask)
            vis = p > 0
            s_hat = float((scale * (np.abs(q[b, h]) @ np.abs(k[b, h]).T))[vis].max()) if vis.any() else 0.0
            l_max = float(np.abs(lse[b, h][np.isfinite(lse[b, h])]).max()) if np.isfinite(lse[b, h]).any() else 0.0
            eps = 4 * U * (d * s_hat + l_max + max(nq, nk) + 16)
            a_ds = p * ((np.abs(do[b, h]) @ np.abs(v[b, h]).T)
                        + (np.abs(do[b, h]) * np.abs(o[b, h])).sum(axis=1, keepdims=True))
            bv[b, h] = eps * (p.T @ np.abs(do[b, h])) + 1e-7
            bk[b, h] = eps * scale * (a_ds.T @ np.abs(q[b, h])) + 1e-7
            bq[b, h] = eps * scale * (a_ds @ np.abs(k[b, h])) + 1e-7
            bds[b, h] = eps * a_ds + 1e-7
            masked[b, h] = ~vis
    if with_ds:
        return (bq, bk, bv), bds, masked
    return bq, bk, bv


def check32(got, want, bounds, what):
    for name, g, w, bd in zip(("dQ", "dK", "dV"), got, want, bounds):
        g = np64(g)
        assert np.isfinite(g).all(), f"{what}: non-finite {name}"
        err = np.abs(g - w)
        worst = np.unravel_index(np.argmax(err - bd), err.shape) if err.size else None
        assert np.all(err <= bd), (f"{what}: {name} err {err[worst]:.3e} > bound {bd[worst]:.3e} "
                                   f"at {worst}")


def run(q, k, v, do, **kw):
    qd, kd, vd, dod = (t.to(DEV) for t in (q, k, v, do))
    o, lse = fa.fa_fwd(qd, kd, vd, **kw)
    got = fa.fa_bwd(dod, qd, kd, vd, o, lse, **kw)
    torch.cuda.synchronize()
    assert all(g.dtype == torch.float32 for g in got)
    return got


SHAPES = [(1, 1), (3, 2), (63, 65), (200, 333), (333, 200), (520, 520)]


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("nq,nk", SHAPES)
def test_fp32_backward_matches_oracle(d, causal, nq, nk):
    B, H = 1, 2
    seed = 7001 * nq + 17 * nk + d + (1 if causal else 0)
    q, k, v, do = (normal((B, H, n, d), torch.float32, seed + i)
                   for i, n in enumerate((nq, nk, nk, nq)))
    scale = 1.0 / math.sqrt(d)
    got = run(q, k, v, do, scale=scale, causal=causal)
    qn, kn, vn, don = np64(q), np64(k), np64(v), np64(do)
    want = oracle.attention_backward(qn, kn, vn, don, scale, causal=causal)
    check32(got, want, grad_bounds(qn, kn, vn, don, scale, causal), f"fp32 d{d} c{causal} {nq}x{nk}")


@pytest.mark.parametrize("causal", [False, True])
def test_fp32_backward_slope_bias_ranges_and_dslopes(causal):
    B, H, nq, nk, d = 2, 3, 300, 330, 128
    q, k, v, do = (normal((B, H, n, d), torch.float32, 7100 + i)
                   for i, n in enumerate((nq, nk, nk, nq)))
    ks, ke = key_ranges(nq, nk, seed=7105, block=64, width=nk // 2, jitter=32)
    ks, ke = ks.clone(), ke.clone()
    ks[7], ke[7] = 100, 100  # an empty row
    slopes = [-0.02, 0.01, -0.05]
    scale = 1.0 / math.sqrt(d)
    qd, kd, vd, dod = (t.to(DEV) for t in (q, k, v, do))
    kw = dict(causal=causal, scale=scale, bias_slopes=slopes, key_start=ks.to(DEV),
              key_end=ke.to(DEV))
    o, lse = fa.fa_fwd(qd, kd, vd, **kw)
    ds = torch.full((H,), float("nan"), dtype=torch.float32, device=DEV)
    got = fa.fa_bwd(dod, qd, kd, vd, o, lse, dslopes=ds, **kw)
    torch.cuda.synchronize()
    mask = dict(bias_slopes=np.float32(slopes).astype(np.float64), key_start=ks.numpy(),
                key_end=ke.numpy())
    qn, kn, vn, don = np64(q), np64(k), np64(v), np64(do)
    *want, dref = oracle.attention_backward(qn, kn, vn, don, scale, causal=causal,
                                            return_dslopes=True, **mask)
    bounds, bds, _ = grad_bounds(qn, kn, vn, don, scale, causal, with_ds=True, **mask)
    check32(got, want, bounds, "fp32 slope+ranges")
    assert np.all(np64(got[0])[:, :, 7] == 0)  # the empty row: no gradient
    # dL/dslope_h = sum over b, i, j of dS |i - j|: the dS bounds times |i - j|, plus the
    # float32 rounding of the sum (each lane adds up to N_q terms, then a wave, workgroup
    # and key-block reduction: at most N_q + N_k + 64 roundings of the running sum)
    dist = np.abs(np.arange(nq)[:, None] - np.arange(nk)[None, :])
    abs_terms = np.zeros(H)
    for b in range(B):
        for h in range(H):
            p = oracle.attention_probabilities(qn, kn, scale, b, h, causal, **mask)
            dp = don[b, h] @ vn[b, h].T
            dsm = p * (dp - (p * dp).sum(axis=1, keepdims=True))
            abs_terms[h] += (np.abs(dsm) * dist).sum()
    tol = (bds * dist).sum(axis=(0, 2, 3)) + 4 * U * (nq + nk + 64) * abs_terms
    err = np.abs(ds.cpu().numpy() - dref)
    assert np.all(err <= tol), (ds.cpu().numpy(), dref, tol)


def test_fp32_backward_bias_tensor_and_dbias():
    # dense dbias, then dbias summed over each broadcast axis set
    B, H, nq, nk, d = 2, 2, 257, 300, 64
    q, k, v, do = (normal((B, H, n, d), torch.float32, 7200 + i)
                   for i, n in enumerate((nq, nk, nk, nq)))
    bias = bias_tensor((1, H, nq, nk), 7205, 2.0, 0.05)
    bias[:, 1, 9] = float("-inf")  # a row with no visible key
    scale = 1.0 / math.sqrt(d)
    qd, kd, vd, dod, bd = (t.to(DEV) for t in (q, k, v, do, bias))
    o, lse = fa.fa_fwd(qd, kd, vd, causal=True, scale=scale, bias=bd)
    dbias = torch.full((B, H, nq, nk), float("nan"), dtype=torch.float32, device=DEV)
    got = fa.fa_bwd(dod, qd, kd, vd, o, lse, causal=True, scale=scale, bias=bd, dbias=dbias)
    torch.cuda.synchronize()
    qn, kn, vn, don, bn = np64(q), np64(k), np64(v), np64(do), bias.double().numpy()
    *want, dref = oracle.attention_backward(qn, kn, vn, don, scale, causal=True, bias=bn,
                                            return_dbias=True)
    bounds, bds, masked = grad_bounds(qn, kn, vn, don, scale, True, with_ds=True, bias=bn)
    check32(got, want, bounds, "fp32 bias tensor")
    g = np64(dbias)
    assert np.isfinite(g).all()
    assert np.all(g[masked] == 0)  # masked entries (and the empty row) exactly zero
    err = np.abs(g - dref)
    assert np.all(err <= bds), float((err - bds).max())
    # dbias summed over broadcast axes (b batches, h heads, i query rows): the sum of the
    # per-element bounds plus the float32 rounding of a sum of n terms; an element whose
    # every summand is masked is exactly zero; a second call gives the same bits
    for axes in ("b", "bh", "i", "bhi"):
        red = tuple(ax for ax, c in enumerate("bhi") if c in axes)
        shape = tuple(1 if i in red else n for i, n in enumerate((B, H, nq, nk)))
        n_terms = int(np.prod([(B, H, nq)[ax] for ax in red]))
        sums = []
        for _ in range(2):
            db = torch.full(shape, float("nan"), dtype=torch.float32, device=DEV)
            got2 = fa.fa_bwd(dod, qd, kd, vd, o, lse, causal=True, scale=scale, bias=bd,
                             dbias=db)
            torch.cuda.synchronize()
            sums.append(db)
        for a, b in zip(got2, got):
            assert torch.equal(a, b), axes  # the gradients do not depend on dbias
        assert torch.equal(sums[0], sums[1]), axes
        g = np64(sums[0])
        ref = dref.sum(axis=red, keepdims=True)
        bound = (bds.sum(axis=red, keepdims=True)
                 + n_terms * 2.0 ** -23 * np.abs(dref).sum(axis=red, keepdims=True))
        assert g.shape == ref.shape and np.isfinite(g).all(), axes
        err = np.abs(g - ref)
        assert np.all(err <= bound), (axes, float((err - bound).max()))
        assert np.all(g[masked.all(axis=red, keepdims=True)] == 0), axes


def test_fp32_backward_c1_workload():
    # the float32 workload (B1 H1 N256 d64, non-causal) through the backward
    w = WORKLOADS[1]
    q, k, v, do = qkv_inputs(w, with_dout=True)
    got = run(q, k, v, do, scale=w.scale, causal=w.causal)
    qn, kn, vn, don = np64(q), np64(k), np64(v), np64(do)
    want = oracle.attention_backward(qn, kn, vn, don, w.scale, causal=w.causal)
    check32(got, want, grad_bounds(qn, kn, vn, don, w.scale, w.causal), "C1 backward")


def test_fp32_backward_is_deterministic_and_phases_agree():
    B, H, n, d = 1, 3, 700, 128
    q, k, v, do = (normal((B, H, n, d), torch.float32, 7300 + i).to(DEV) for i in range(4))
    o, lse = fa.fa_fwd(q, k, v, causal=True)
    a = fa.fa_bwd(do, q, k, v, o, lse, causal=True)
    b = fa.fa_bwd(do, q, k, v, o, lse, causal=True)
    ws = torch.empty(fa.fa_bwd_workspace_bytes(B, H, n, n, d), dtype=torch.uint8, device=DEV)
    grads = tuple(torch.empty_like(q) for _ in range(3))
    for ph in (fa.FA_BWD_PREP, fa.FA_BWD_DKDV, fa.FA_BWD_DQ):
        fa.fa_bwd(do, q, k, v, o, lse, causal=True, grads=grads, workspace=ws, phases=ph)
    torch.cuda.synchronize()
    for x, y, z in zip(a, b, grads):
        assert torch.equal(x, y) and torch.equal(x, z)


@pytest.mark.parametrize("causal,layout", [(True, "head"), (False, "batch_head")])
def test_fp32_block_bitmap_forward_and_backward(causal, layout):
    # float32 inputs apply a block bitmap as a mask (forward, split forward, backward)
    B, H, nq, nk, d, bq, bk = 2, 2, 300, 330, 64, 64, 128
    q, k, v, do = (normal((B, H, n, d), torch.float32, 7400 + i)
                   for i, n in enumerate((nq, nk, nk, nq)))
    nbq, nbk = -(-nq // bq), -(-nk // bk)
    shape = {"head": (H, nbq, nbk), "batch_head": (B, H, nbq, nbk)}[layout]
    bm = (np.random.default_rng(7405).random(shape) < 0.6).astype(np.uint8)
    scale = 1.0 / math.sqrt(d)
    qd, kd, vd, dod = (t.to(DEV) for t in (q, k, v, do))
    kw = dict(causal=causal, scale=scale, block_mask=(torch.from_numpy(bm).to(DEV), bq, bk))
    o, lse = fa.fa_fwd(qd, kd, vd, **kw)
    o2, lse2 = fa.fa_fwd_split(qd, kd, vd, n_split=3, **kw)
    got = fa.fa_bwd(dod, qd, kd, vd, o, lse, **kw)
    torch.cuda.synchronize()
    qn, kn, vn, don = np64(q), np64(k), np64(v), np64(do)
    mask = dict(block_mask=(bm, bq, bk))
    o_ref, lse_ref = oracle.attention_forward(qn, kn, vn, scale, causal=causal, **mask)
    what = f"fp32 bitmap {layout} c{causal}"
    assert_fwd_close(np64(o), np64(lse), o_ref, lse_ref, torch.float32, what)
    assert_fwd_close(np64(o2), np64(lse2), o_ref, lse_ref, torch.float32, what + " split")
    want = oracle.attention_backward(qn, kn, vn, don, scale, causal=causal, **mask)
    check32(got, want, grad_bounds(qn, kn, vn, don, scale, causal, **mask), what)
