"""GPU backward parity (recomputation from O and LSE) against the fp64 oracle gradients."""

import math

import numpy as np
import pytest
import torch

import oracle
from synth import WORKLOADS, key_ranges, normal, qkv_inputs
from tests.util import GRAD_TOL, np64

pytestmark = pytest.mark.gpu

fa = pytest.importorskip("exact_io_aware_flash_amd")
DEV = "cuda:0"


def fwd_bwd(q, k, v, do, grad_dtype=torch.float32, **kw):
    q, k, v, do = (t.to(DEV) for t in (q, k, v, do))
    o, lse = fa.fa_fwd(q, k, v, **kw)
    dq, dk, dv = fa.fa_bwd(do, q, k, v, o, lse, grad_dtype=grad_dtype, **kw)
    torch.cuda.synchronize()
    return dq, dk, dv


def check_grads(got, want, what, tol=GRAD_TOL, rel=0.0):
    for name, g, w in zip(("dQ", "dK", "dV"), got, want):
        g = np64(g)
        assert np.isfinite(g).all(), f"{what}: non-finite {name}"
        err = np.abs(g - w) - rel * np.abs(w)
        worst = float(err.max()) if err.size else 0.0
        assert worst <= tol, f"{what}: {name} max err {worst:.3e} > {tol}"


SHAPES = [(1, 1), (3, 2), (63, 65), (128, 128), (200, 333), (333, 200), (520, 520)]


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float16])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("nq,nk", SHAPES)
def test_small_shapes(dtype, d, causal, nq, nk):
    B, H = 1, 2
    seed = 10007 * nq + 31 * nk + d + (1 if causal else 0)
    q = normal((B, H, nq, d), dtype, seed)
    k = normal((B, H, nk, d), dtype, seed + 1)
    v = normal((B, H, nk, d), dtype, seed + 2)
    do = normal((B, H, nq, d), dtype, seed + 3)
    scale = 1.0 / math.sqrt(d)
    got = fwd_bwd(q, k, v, do, scale=scale, causal=causal)
    want = oracle.attention_backward(np64(q), np64(k), np64(v), np64(do), scale, causal=causal)
    check_grads(got, want, f"{dtype} d{d} c{causal} {nq}x{nk}")


@pytest.mark.parametrize("dtype,d", [(torch.bfloat16, 128), (torch.float16, 64)])
@pytest.mark.parametrize("causal", [False, True])
def test_bias_and_key_ranges(dtype, d, causal):
    B, H, nq, nk = 1, 3, 520, 450
    q, k, v, do = (normal((B, H, n, d), dtype, 70 + i)
                   for i, n in enumerate((nq, nk, nk, nq)))
    ks, ke = key_ranges(nq, nk, seed=75, block=64, width=nk // 2, jitter=32)
    ks, ke = ks.clone(), ke.clone()
    ks[3], ke[3] = -40, 5
    ks[4], ke[4] = 300, 300  # empty row
    ks[500], ke[500] = 0, 99999
    slopes = [-0.1 / 64, 0.03, -0.02]
    scale = 1.0 / math.sqrt(d)
    got = fwd_bwd(q, k, v, do, scale=scale, causal=causal, bias_slopes=slopes,
                  key_start=ks.to(DEV), key_end=ke.to(DEV))
    want = oracle.attention_backward(np64(q), np64(k), np64(v), np64(do), scale, causal=causal,
                                     bias_slopes=np.float32(slopes).astype(np.float64),
                                     key_start=ks.numpy(), key_end=ke.numpy())
    check_grads(got, want, f"bias+range {dtype} d{d} c{causal}")


def test_low_precision_gradient_outputs():
    # gradients written in bf16: the bound adds the bf16 rounding of each value
    B, H, n, d = 1, 2, 300, 128
    q, k, v, do = (normal((B, H, n, d), torch.bfloat16, 80 + i) for i in range(4))
    got = fwd_bwd(q, k, v, do, grad_dtype=torch.bfloat16, causal=True)
    assert all(g.dtype == torch.bfloat16 for g in got)
    want = oracle.attention_backward(np64(q), np64(k), np64(v), np64(do), 1 / math.sqrt(d),
                                     causal=True)
    check_grads(got, want, "bf16 grads", tol=GRAD_TOL, rel=2.0 ** -8)


def test_backward_is_deterministic():
    B, H, n, d = 1, 4, 700, 128
    q, k, v, do = (normal((B, H, n, d), torch.bfloat16, 90 + i) for i in range(4))
    a = fwd_bwd(q, k, v, do, causal=True)
    b = fwd_bwd(q, k, v, do, causal=True)
    for x, y in zip(a, b):
        assert torch.equal(x, y)


def test_full_causal_bf16_n8192_backward():
    # the full fwd+bwd workload; the oracle checks two whole (b, h) heads
    w = WORKLOADS[5]
    q, k, v, do = qkv_inputs(w)
    dq, dk, dv = fwd_bwd(q, k, v, do, scale=w.scale, causal=True)
    for g in (dq, dk, dv):
        assert torch.isfinite(g).all()
    for (b, h) in ((0, 0), (1, 13)):
        one = lambda t: np64(t[b:b + 1, h:h + 1])  # noqa: E731
        want = oracle.attention_backward(one(q), one(k), one(v), one(do), w.scale, causal=True,
                                         max_chunk_elems=1 << 25)
        got = (dq[b:b + 1, h:h + 1], dk[b:b + 1, h:h + 1], dv[b:b + 1, h:h + 1])
        check_grads(got, want, f"{w.name} b{b} h{h}")


@pytest.mark.parametrize("dtype,d", [(torch.bfloat16, 128), (torch.float16, 64)])
@pytest.mark.parametrize("causal,ranged,per_head", [(True, False, True), (False, True, False),
                                                    (True, True, True)])
def test_slope_gradient(dtype, d, causal, ranged, per_head):
    # dL/dslope = sum dS |i - j| (per head, or over all heads for one shared slope);
    # tolerance 1e-2 of sum |dS| |i - j|, the scale of the terms being added
    B, H, nq, nk = 2, 3, 300, 330
    q, k, v, do = (normal((B, H, n, d), dtype, 8800 + i) for i, n in enumerate((nq, nk, nk, nq)))
    slopes = [-0.02, 0.01, -0.05] if per_head else [-0.03]
    kw = dict(causal=causal, scale=1.0 / math.sqrt(d), bias_slopes=slopes)
    if ranged:
        ks, ke = key_ranges(nq, nk, seed=8805, block=64, width=nk // 2, jitter=32)
        kw.update(key_start=ks.to(DEV), key_end=ke.to(DEV))
    qd, kd, vd, dod = (t.to(DEV) for t in (q, k, v, do))
    o, lse = fa.fa_fwd(qd, kd, vd, **kw)
    ds = torch.full((len(slopes),), float("nan"), dtype=torch.float32, device=DEV)
    got = fa.fa_bwd(dod, qd, kd, vd, o, lse, dslopes=ds, **kw)
    torch.cuda.synchronize()
    ref_kw = dict(causal=causal, bias_slopes=np.float32(slopes).astype(np.float64))
    if ranged:
        ref_kw.update(key_start=ks.numpy(), key_end=ke.numpy())
    *want, dref = oracle.attention_backward(np64(q), np64(k), np64(v), np64(do), kw["scale"],
                                            return_dslopes=True, **ref_kw)
    check_grads(got, want, "grads with dslopes")
    # scale of the terms: sum |dS| |i - j| from the oracle's probabilities
    tot = np.zeros(H)
    for b in range(B):
        for h in range(H):
            p = oracle.attention_probabilities(np64(q), np64(k), kw["scale"], b, h, causal,
                                               bias_slopes=ref_kw["bias_slopes"],
                                               key_start=ref_kw.get("key_start"),
                                               key_end=ref_kw.get("key_end"))
            dp = np64(do)[b, h] @ np64(v)[b, h].T
            dsm = p * (dp - (p * dp).sum(axis=1, keepdims=True))
            dist = np.abs(np.arange(nq)[:, None] - np.arange(nk)[None, :])
            tot[h] += np.abs(dsm * dist).sum()
    scale_terms = tot if per_head else tot.sum(keepdims=True)
    err = np.abs(ds.cpu().numpy() - dref)
    assert np.all(err <= 1e-2 * scale_terms + 1e-4), (ds.cpu().numpy(), dref, scale_terms)
