"""GPU parity of the float32 bias-tensor path (FA_BIAS_TENSOR): forward, split forward and
backward with dbias, against the float64 oracle on the same seeded inputs.

Source: scifaro.com related-papers page for FlashMask (arXiv 2410.01359), the abstract on
attention with an additive bias matrix. Tolerances as for the other parity tests: O within
1e-5 (float32 inputs) or 2e-2 (bf16/fp16), LSE within 1e-3 relative, dQ, dK, dV within
2e-2 absolute (float32 gradients of 16-bit inputs).

dbias = dS = P o (dP - D) has a bound of its own, derived from the arithmetic: the
backward takes D_i = sum_c dO_ic O_ic from the stored 16-bit O, whose entries differ from
the exact ones by the rounding of the probabilities before P V (2^-9 relative each) and of
the stored value (2^-9), so |dO_i| . |dO - O| <= 2^-8 sum_c |dO_ic| (P |V|)_ic =: 2^-8 A_i.
Every other step is float32 (relative 1e-6 scale), so per element
    |d dbias_ij| <= P_ij (2^-8 A_i + 1e-3) + 1e-6,
with P the oracle's probabilities (large where a bias makes the softmax peaky, which is
where this term exceeds a flat 2e-2).
"""

import math

import numpy as np
import pytest
import torch

import oracle
from synth import WORKLOADS, bias_tensor, key_ranges, normal, qkv_inputs, seed_for
from tests.util import GRAD_TOL, assert_fwd_close, np64, sample_rows

pytestmark = pytest.mark.gpu

fa = pytest.importorskip("exact_io_aware_flash_amd")
DEV = "cuda:0"


def bias_shape(kind, B, H, nq, nk):
    return {"full": (B, H, nq, nk), "head": (1, H, nq, nk), "key": (B, 1, 1, nk),
            "rows": (1, 1, nq, nk)}[kind]


def strided(b):
    """The same values in a buffer whose rows are 3 floats longer (row stride nk + 3)."""
    big = torch.full(b.shape[:-1] + (b.shape[-1] + 3,), 7.0, dtype=b.dtype, device=b.device)
    big[..., :b.shape[-1]] = b
    return big[..., :b.shape[-1]]


FWD_CASES = [
    # dtype, d, causal, nq, nk, bias kind, -inf fraction, key ranges, row-strided buffer
    (torch.bfloat16, 128, True, 300, 300, "full", 0.0, False, False),
    (torch.bfloat16, 128, False, 200, 333, "head", 0.1, False, True),
    (torch.float16, 64, True, 257, 513, "key", 0.0, False, False),
    (torch.float16, 64, False, 129, 70, "full", 0.05, True, True),
    (torch.bfloat16, 128, True, 1000, 1000, "rows", 0.0, True, False),
    (torch.bfloat16, 64, True, 64, 64, "full", 0.0, False, False),
    (torch.float16, 128, False, 1, 1, "full", 0.0, False, False),
    (torch.float32, 128, True, 200, 250, "full", 0.1, False, True),
    (torch.float32, 64, False, 100, 77, "key", 0.0, True, False),
]


@pytest.mark.parametrize("dtype,d,causal,nq,nk,kind,ninf,ranged,stride", FWD_CASES)
def test_forward_matches_oracle(dtype, d, causal, nq, nk, kind, ninf, ranged, stride):
    B, H = 2, 3
    seed = 900 + nq + 7 * nk + d
    q, k, v = (normal((B, H, n, d), dtype, seed + i) for i, n in enumerate((nq, nk, nk)))
    bias = bias_tensor(bias_shape(kind, B, H, nq, nk), seed + 5, 2.0, ninf)
    if kind == "full" and nq > 2:
        bias[0, 1, 2] = float("-inf")  # a row whose every entry is masked by the bias
    kw = {}
    ks = ke = None
    if ranged:
        ks, ke = key_ranges(nq, nk, seed=seed + 6, block=64, width=max(nk // 2, 1), jitter=16)
        kw = dict(key_start=ks.to(DEV), key_end=ke.to(DEV))
    bd = bias.to(DEV)
    if stride:
        bd = strided(bd)
    scale = 1.0 / math.sqrt(d)
    o, lse = fa.fa_fwd(q.to(DEV), k.to(DEV), v.to(DEV), causal=causal, scale=scale, bias=bd, **kw)
    torch.cuda.synchronize()
    o_ref, lse_ref = oracle.attention_forward(
        np64(q), np64(k), np64(v), scale, causal=causal, bias=bias.double().numpy(),
        key_start=None if ks is None else ks.numpy(), key_end=None if ke is None else ke.numpy())
    assert_fwd_close(np64(o), np64(lse), o_ref, lse_ref, dtype,
                     f"bias {kind} {dtype} d{d} c{causal} {nq}x{nk}")


@pytest.mark.parametrize("d,nq,nk,n_split", [(128, 1, 2000, 4), (128, 16, 4100, 0),
                                              (128, 64, 777, 3), (64, 5, 1500, 0),
                                              (64, 64, 1000, 2)])
def test_split_forward_matches_oracle(d, nq, nk, n_split):
    B, H = 2, 4
    dtype = torch.bfloat16
    q, k, v = (normal((B, H, n, d), dtype, 950 + i) for i, n in enumerate((nq, nk, nk)))
    bias = bias_tensor((B, H, nq, nk), 955, 1.5, 0.02)
    assert fa.fa_fwd_split_count(B, H, nq, nk, d, n_split) > 1
    o, lse = fa.fa_fwd_split(q.to(DEV), k.to(DEV), v.to(DEV), causal=True, bias=bias.to(DEV),
                             n_split=n_split)
    torch.cuda.synchronize()
    o_ref, lse_ref = oracle.attention_forward(np64(q), np64(k), np64(v), 1 / math.sqrt(d),
                                              causal=True, bias=bias.double().numpy())
    assert_fwd_close(np64(o), np64(lse), o_ref, lse_ref, dtype, f"split bias {nq}x{nk}")


def check(got, want, names, what):
    for name, g, w in zip(names, got, want):
        g = np64(g)
        assert np.isfinite(g).all(), f"{what}: non-finite {name}"
        err = float(np.abs(g - w).max()) if g.size else 0.0
        assert err <= GRAD_TOL, f"{what}: {name} max err {err:.3e} > {GRAD_TOL}"


def dbias_tol(q, k, v, do, scale, causal, bias, ks, ke):
    """Per-element bound on |dbias - dS| (module docstring), [B, H, N_q, N_k], and the
    entries the oracle masks (probability exactly 0)."""
    B, H, nq, _ = q.shape
    nk = k.shape[2]
    tol = np.empty((B, H, nq, nk))
    masked = np.empty((B, H, nq, nk), dtype=bool)
    for b in range(B):
        for h in range(H):
            p = oracle.attention_probabilities(q, k, scale, b, h, causal, key_start=ks,
                                               key_end=ke, bias=bias)
            a = (np.abs(do[b, h]) * (p @ np.abs(v[b, h]))).sum(axis=1)
            tol[b, h] = p * (2.0 ** -8 * a[:, None] + 1e-3) + 1e-6
            masked[b, h] = p == 0
    return tol, masked


def check_dbias(got, want, tol_masked, what):
    tol, masked = tol_masked
    g = np64(got)
    assert np.isfinite(g).all(), f"{what}: non-finite dbias"
    err = np.abs(g - want)
    worst = np.unravel_index(np.argmax(err - tol), err.shape)
    assert np.all(err <= tol), (f"{what}: |d dbias| {err[worst]:.3e} > {tol[worst]:.3e} "
                                f"at {tuple(int(x) for x in worst)}")
    # masked entries are exactly zero (the library clears what it skips)
    assert np.all(g[masked] == 0), f"{what}: {int((g[masked] != 0).sum())} masked entries != 0"


def plant_empty_rows(bias, kind):
    """Set -inf over whole rows of the bias, so that those query rows see no key (their
    forward gives O = 0 and LSE = -inf; their probabilities, gradients and dbias are 0).
    "full" / "head": rows 0, 5, 64 and 130 of head 1 (inside fully visible tiles when
    nothing else masks them); "key" ([B, 1, 1, N_k]): every row of batch 1."""
    if kind in ("full", "head"):
        for r in (0, 5, 64, 130):
            if r < bias.shape[2]:
                bias[:, 1, r] = float("-inf")
    elif kind == "key":
        bias[1] = float("-inf")
    else:
        raise ValueError(kind)


BWD_CASES = [
    # dtype, d, causal, nq, nk, bias kind, -inf fraction, key ranges, rows emptied by the bias
    (torch.bfloat16, 128, True, 300, 300, "full", 0.0, False, False),
    (torch.float16, 64, False, 200, 333, "head", 0.1, False, False),
    (torch.bfloat16, 64, True, 257, 513, "key", 0.0, True, False),
    (torch.float16, 128, True, 130, 70, "full", 0.05, False, False),
    (torch.bfloat16, 128, False, 3, 1, "rows", 0.0, False, False),
    # rows whose every entry is -inf: in fully visible tiles (non-causal, no ranges) ...
    (torch.bfloat16, 128, False, 300, 300, "full", 0.0, False, True),
    (torch.float16, 64, False, 200, 333, "head", 0.02, False, True),
    # ... under key ranges, and a whole batch masked (causal, partial tiles)
    (torch.bfloat16, 128, False, 257, 300, "head", 0.0, True, True),
    (torch.float16, 128, True, 130, 200, "key", 0.0, False, True),
]


@pytest.mark.parametrize("dtype,d,causal,nq,nk,kind,ninf,ranged,empty", BWD_CASES)
def test_backward_and_dbias_match_oracle(dtype, d, causal, nq, nk, kind, ninf, ranged, empty):
    B, H = 2, 2
    seed = 970 + nq + 3 * nk + d
    q, k, v, do = (normal((B, H, n, d), dtype, seed + i) for i, n in enumerate((nq, nk, nk, nq)))
    bias = bias_tensor(bias_shape(kind, B, H, nq, nk), seed + 5, 2.0, ninf)
    if empty:
        plant_empty_rows(bias, kind)
    kw = {}
    ks = ke = None
    if ranged:
        ks, ke = key_ranges(nq, nk, seed=seed + 6, block=64, width=max(nk // 2, 1), jitter=16)
        kw = dict(key_start=ks.to(DEV), key_end=ke.to(DEV))
    scale = 1.0 / math.sqrt(d)
    qd, kd, vd, dod, bd = (t.to(DEV) for t in (q, k, v, do, bias))
    o, lse = fa.fa_fwd(qd, kd, vd, causal=causal, scale=scale, bias=bd, **kw)
    dbias = torch.full((B, H, nq, nk), float("nan"), dtype=torch.float32, device=DEV)
    dq, dk, dv = fa.fa_bwd(dod, qd, kd, vd, o, lse, causal=causal, scale=scale, bias=bd,
                           dbias=dbias, **kw)
    torch.cuda.synchronize()
    want = oracle.attention_backward(
        np64(q), np64(k), np64(v), np64(do), scale, causal=causal, bias=bias.double().numpy(),
        key_start=None if ks is None else ks.numpy(), key_end=None if ke is None else ke.numpy(),
        return_dbias=True)
    what = f"bias {kind} {dtype} d{d} c{causal} {nq}x{nk}" + (" empty rows" if empty else "")
    if empty:
        # the planted rows are empty in the forward and give exact zeros in the backward
        lse_np = np64(lse)
        ref_empty = ~np.isfinite(oracle.attention_forward(
            np64(q), np64(k), np64(v), scale, causal=causal, bias=bias.double().numpy(),
            key_start=None if ks is None else ks.numpy(),
            key_end=None if ke is None else ke.numpy())[1])
        assert ref_empty.any(), what
        assert np.all(np.isneginf(lse_np[ref_empty])), what
        assert np.all(np64(dq)[ref_empty] == 0), what
        assert np.all(np64(dbias)[ref_empty] == 0), what
    check((dq, dk, dv), want[:3], ("dQ", "dK", "dV"), what)
    ksn = None if ks is None else ks.numpy()
    ken = None if ke is None else ke.numpy()
    check_dbias(dbias, want[3], dbias_tol(np64(q), np64(k), np64(v), np64(do), scale, causal,
                                          bias.double().numpy(), ksn, ken), what)
    # without dbias the gradients are the same bits
    dq2, dk2, dv2 = fa.fa_bwd(dod, qd, kd, vd, o, lse, causal=causal, scale=scale, bias=bd, **kw)
    torch.cuda.synchronize()
    for a, b in ((dq, dq2), (dk, dk2), (dv, dv2)):
        assert torch.equal(a, b), what


RED_CASES = [
    # dtype, d, causal, nq, nk, summed axes (b batches, h heads, i query rows), -inf
    # fraction, key ranges
    (torch.bfloat16, 128, True, 300, 300, "b", 0.0, False),
    (torch.float16, 64, False, 200, 333, "h", 0.05, False),
    (torch.bfloat16, 128, False, 257, 300, "bh", 0.0, True),
    (torch.bfloat16, 64, True, 257, 513, "i", 0.0, False),
    (torch.float16, 128, True, 130, 200, "bhi", 0.0, True),
    (torch.bfloat16, 128, False, 3, 1, "hi", 0.0, False),
    (torch.float16, 64, True, 200, 70, "bi", 0.1, False),
]


@pytest.mark.parametrize("dtype,d,causal,nq,nk,axes,ninf,ranged", RED_CASES)
def test_dbias_summed_over_broadcast_axes(dtype, d, causal, nq, nk, axes, ninf, ranged):
    # a bias broadcast over some axes (size 1 there): a dbias of the bias's own shape
    # receives dS summed over those axes. Bound: the sum of the per-element bounds plus
    # the float32 rounding of a sum of n terms (n 2^-23 times the sum of |dS|).
    B, H = 2, 3
    seed = 4100 + nq + 7 * nk + d
    q, k, v, do = (normal((B, H, n, d), dtype, seed + i) for i, n in enumerate((nq, nk, nk, nq)))
    shape = (1 if "b" in axes else B, 1 if "h" in axes else H, 1 if "i" in axes else nq, nk)
    bias = bias_tensor(shape, seed + 5, 2.0, ninf)
    kw = {}
    ks = ke = None
    if ranged:
        ks, ke = key_ranges(nq, nk, seed=seed + 6, block=64, width=max(nk // 2, 1), jitter=16)
        kw = dict(key_start=ks.to(DEV), key_end=ke.to(DEV))
    scale = 1.0 / math.sqrt(d)
    qd, kd, vd, dod, bd = (t.to(DEV) for t in (q, k, v, do, bias))
    o, lse = fa.fa_fwd(qd, kd, vd, causal=causal, scale=scale, bias=bd, **kw)
    dbias = torch.full(shape, float("nan"), dtype=torch.float32, device=DEV)
    dq, dk, dv = fa.fa_bwd(dod, qd, kd, vd, o, lse, causal=causal, scale=scale, bias=bd,
                           dbias=dbias, **kw)
    torch.cuda.synchronize()
    ksn = None if ks is None else ks.numpy()
    ken = None if ke is None else ke.numpy()
    want = oracle.attention_backward(np64(q), np64(k), np64(v), np64(do), scale, causal=causal,
                                     bias=bias.double().numpy(), key_start=ksn, key_end=ken,
                                     return_dbias=True)
    what = f"dbias summed over {axes}: {dtype} d{d} c{causal} {nq}x{nk}"
    check((dq, dk, dv), want[:3], ("dQ", "dK", "dV"), what)
    red = tuple(ax for ax, c in enumerate("bhi") if c in axes)
    n_terms = int(np.prod([(B, H, nq)[ax] for ax in red]))
    tol, masked = dbias_tol(np64(q), np64(k), np64(v), np64(do), scale, causal,
                            bias.double().numpy(), ksn, ken)
    ref = want[3].sum(axis=red, keepdims=True)
    bound = (tol.sum(axis=red, keepdims=True)
             + n_terms * 2.0 ** -23 * np.abs(want[3]).sum(axis=red, keepdims=True))
    g = np64(dbias)
    assert g.shape == ref.shape and np.isfinite(g).all(), what
    err = np.abs(g - ref)
    worst = np.unravel_index(np.argmax(err - bound), err.shape)
    assert np.all(err <= bound), (f"{what}: {err[worst]:.3e} > {bound[worst]:.3e} at "
                                  f"{tuple(int(x) for x in worst)}")
    # an element whose every summand is masked is exactly zero
    assert np.all(g[masked.all(axis=red, keepdims=True)] == 0), what
    # deterministic, and the gradients are the same bits as without dbias
    dbias2 = torch.full(shape, float("nan"), dtype=torch.float32, device=DEV)
    g2 = fa.fa_bwd(dod, qd, kd, vd, o, lse, causal=causal, scale=scale, bias=bd, dbias=dbias2,
                   **kw)
    g3 = fa.fa_bwd(dod, qd, kd, vd, o, lse, causal=causal, scale=scale, bias=bd, **kw)
    torch.cuda.synchronize()
    assert torch.equal(dbias, dbias2), what
    for a, b2, b3 in zip((dq, dk, dv), g2, g3):
        assert torch.equal(a, b2) and torch.equal(a, b3), what


def test_dbias_shape_is_checked():
    q = torch.zeros((2, 3, 64, 64), dtype=torch.bfloat16, device=DEV)
    o, lse = fa.fa_fwd(q, q, q)
    bias = torch.zeros((1, 3, 64, 64), dtype=torch.float32, device=DEV)
    for shape in ((2, 2, 64, 64), (1, 3, 64, 63), (3, 64, 64)):
        with pytest.raises(ValueError):
            fa.fa_bwd(q, q, q, q, o, lse, bias=bias,
                      dbias=torch.zeros(shape, dtype=torch.float32, device=DEV))


def test_full_size_dbias_summed_over_batch_equals_dense_sum():
    # the bf16 B2 H8 N8192 d128 workload with key ranges and a bias shared over the batch
    # ([1, H, N, N]): dbias of that shape equals the dense [B, H, N, N] dbias (whose parity
    # the tests above establish) summed over the batch, up to one float32 rounding
    w = WORKLOADS[4]
    q, k, v, do = (t.to(DEV) for t in qkv_inputs(w, with_dout=True))
    ks, ke = key_ranges(w.N_q, w.N_k, seed_for(w.wid, 9), block=128, width=w.N_k // 2, jitter=64)
    bias = bias_tensor((1, w.H, w.N_q, w.N_k), seed_for(w.wid, 10), 1.0).to(DEV)
    kw = dict(causal=w.causal, scale=w.scale, bias=bias, key_start=ks.to(DEV),
              key_end=ke.to(DEV))
    o, lse = fa.fa_fwd(q, k, v, **kw)
    dense = torch.empty((w.B, w.H, w.N_q, w.N_k), dtype=torch.float32, device=DEV)
    g1 = fa.fa_bwd(do, q, k, v, o, lse, dbias=dense, **kw)
    summed = torch.full((1, w.H, w.N_q, w.N_k), float("nan"), dtype=torch.float32, device=DEV)
    g2 = fa.fa_bwd(do, q, k, v, o, lse, dbias=summed, **kw)
    torch.cuda.synchronize()
    for a, b in zip(g1, g2):
        assert torch.equal(a, b)
    for h in range(w.H):
        ref = dense[0, h].double() + dense[1, h].double()
        err = (summed[0, h].double() - ref).abs()
        bound = 2.0 ** -23 * (dense[0, h].double().abs() + dense[1, h].double().abs())
        assert bool((err <= bound).all()), f"head {h}: {float((err - bound).max()):.3e}"
    del dense, summed


def test_zero_bias_agrees_with_no_bias():
    # an all-zero bias tensor gives the unbiased result (the two paths round the scores
    # differently: scaled before the row max here, after it without a bias)
    B, H, n, d = 1, 2, 384, 128
    q, k, v = (normal((B, H, n, d), torch.bfloat16, 990 + i) for i in range(3))
    zero = torch.zeros((1, 1, n, n), dtype=torch.float32, device=DEV)
    o1, l1 = fa.fa_fwd(q.to(DEV), k.to(DEV), v.to(DEV), causal=True, bias=zero)
    o0, l0 = fa.fa_fwd(q.to(DEV), k.to(DEV), v.to(DEV), causal=True)
    torch.cuda.synchronize()
    assert float((o1.float() - o0.float()).abs().max()) <= 2e-2
    assert float((l1 - l0).abs().max()) <= 1e-4


def test_full_size_shared_bias_sampled():
    # the bf16 B2 H8 N8192 d128 workload with key ranges and a per-head bias shared over
    # the batch ([1, H, N, N], 2.1 GB): sampled rows of the forward, and one whole head of
    # the backward (dQ, dK, dV, dbias) against the oracle
    w = WORKLOADS[4]
    q, k, v, do = qkv_inputs(w, with_dout=True)
    ks, ke = key_ranges(w.N_q, w.N_k, seed_for(w.wid, 9), block=128, width=w.N_k // 2, jitter=64)
    bias = bias_tensor((1, w.H, w.N_q, w.N_k), seed_for(w.wid, 10), 1.0)
    qd, kd, vd, dod, bd = (t.to(DEV) for t in (q, k, v, do, bias))
    ksd, ked = ks.to(DEV), ke.to(DEV)
    o, lse = fa.fa_fwd(qd, kd, vd, causal=w.causal, scale=w.scale, bias=bd, key_start=ksd,
                       key_end=ked)
    torch.cuda.synchronize()
    rows = sample_rows(w.N_q, 16, 4011)
    bnp = bias.numpy()
    for (b, h) in ((0, 0), (1, 5)):
        o_ref, l_ref = oracle.attention_forward_rows(
            np64(q), np64(k), np64(v), w.scale, rows, b, h, causal=w.causal,
            key_start=ks.numpy(), key_end=ke.numpy(), bias=bnp)
        assert_fwd_close(np64(o[b, h][rows]), np64(lse[b, h][rows]), o_ref, l_ref, w.torch_dtype,
                         f"full-size bias b{b} h{h}")
    dbias = torch.empty((w.B, w.H, w.N_q, w.N_k), dtype=torch.float32, device=DEV)
    dq, dk, dv = fa.fa_bwd(dod, qd, kd, vd, o, lse, causal=w.causal, scale=w.scale, bias=bd,
                           dbias=dbias, key_start=ksd, key_end=ked)
    torch.cuda.synchronize()
    b, h = 1, 3
    one = lambda t: t[b:b + 1, h:h + 1]  # noqa: E731
    want = oracle.attention_backward(
        np64(one(q)), np64(one(k)), np64(one(v)), np64(one(do)), w.scale, causal=w.causal,
        bias=bnp[:, h:h + 1], key_start=ks.numpy(), key_end=ke.numpy(), return_dbias=True)
    check((one(dq), one(dk), one(dv)), want[:3], ("dQ", "dK", "dV"), "full-size bias backward")
    check_dbias(one(dbias), want[3],
                dbias_tol(np64(one(q)), np64(one(k)), np64(one(v)), np64(one(do)), w.scale,
                          w.causal, bnp[:, h:h + 1], ks.numpy(), ke.numpy()),
                "full-size bias backward")


def test_dbias_by_phases_equals_one_call():
    # the dK/dV phase alone writes dbias; the dQ phase leaves it untouched
    B, H, n, d = 1, 2, 200, 64
    q, k, v, do = (normal((B, H, n, d), torch.float16, 1990 + i) for i in range(4))
    bias = bias_tensor((B, 1, n, n), 1995, 1.0, 0.05).to(DEV)
    qd, kd, vd, dod = (t.to(DEV) for t in (q, k, v, do))
    o, lse = fa.fa_fwd(qd, kd, vd, causal=True, bias=bias)
    db1 = torch.full((B, H, n, n), float("nan"), dtype=torch.float32, device=DEV)
    g1 = fa.fa_bwd(dod, qd, kd, vd, o, lse, causal=True, bias=bias, dbias=db1)
    ws = torch.empty(fa.fa_bwd_workspace_bytes(B, H, n, n, d), dtype=torch.uint8, device=DEV)
    db2 = torch.full((B, H, n, n), float("nan"), dtype=torch.float32, device=DEV)
    grads = tuple(torch.empty((B, H, n, d), dtype=torch.float32, device=DEV) for _ in range(3))
    fa.fa_bwd(dod, qd, kd, vd, o, lse, causal=True, bias=bias, dbias=db2, grads=grads,
              workspace=ws, phases=fa.FA_BWD_PREP | fa.FA_BWD_DQ)
    torch.cuda.synchronize()
    assert torch.isnan(db2).all()  # no dK/dV phase: dbias not touched
    fa.fa_bwd(dod, qd, kd, vd, o, lse, causal=True, bias=bias, dbias=db2, grads=grads,
              workspace=ws, phases=fa.FA_BWD_DKDV)
    torch.cuda.synchronize()
    assert torch.equal(db1, db2)
    for a, b in zip(g1, grads):
        assert torch.equal(a, b)


def test_dbias_beyond_2_31_elements_matches_the_head_alone():
    # B2 H16 N8192: dbias holds 2^31 + 2^27 elements (8.6 GB), so the last heads' entries
    # sit past 32-bit offsets; head (1, 15) must equal the same head computed alone (a
    # call with small offsets, whose parity the oracle tests above establish)
    B, H, n, d = 2, 16, 8192, 64
    q, k, v, do = (normal((B, H, n, d), torch.bfloat16, 2990 + i).to(DEV) for i in range(4))
    bias = bias_tensor((1, 1, n, n), 2995, 1.0).to(DEV)
    o, lse = fa.fa_fwd(q, k, v, causal=True, bias=bias)
    dbias = torch.empty((B, H, n, n), dtype=torch.float32, device=DEV)
    dq, dk, dv = fa.fa_bwd(do, q, k, v, o, lse, causal=True, bias=bias, dbias=dbias)
    torch.cuda.synchronize()
    one = lambda t: t[1:2, 15:16].contiguous()  # noqa: E731
    o1, lse1 = fa.fa_fwd(one(q), one(k), one(v), causal=True, bias=bias)
    db1 = torch.empty((1, 1, n, n), dtype=torch.float32, device=DEV)
    g1 = fa.fa_bwd(one(do), one(q), one(k), one(v), o1, lse1, causal=True, bias=bias, dbias=db1)
    torch.cuda.synchronize()
    assert torch.equal(o1, one(o)) and torch.equal(lse1, one(lse))
    assert torch.equal(db1, dbias[1:2, 15:16])
    for a, b in zip(g1, (dq, dk, dv)):
        assert torch.equal(a, one(b))
    del dbias


SPARSE_BIAS_CASES = [
    # dtype, d, causal, nq, nk, bq, bk, density, layout, dbias: "dense", "rows" (summed over
    # query rows), the summed axes (b batches, h heads, i query rows) or None. With a
    # bitmap per (b, h) the members of a summed dbias visit different tiles.
    (torch.bfloat16, 128, True, 300, 330, 64, 64, 0.6, "head", "dense"),
    (torch.float16, 64, False, 257, 520, 128, 64, 0.5, "batch_head", "rows"),
    (torch.bfloat16, 128, False, 200, 700, 64, 192, 0.4, "shared", None),
    (torch.bfloat16, 128, True, 300, 330, 64, 64, 0.6, "batch_head", "b"),
    (torch.float16, 64, False, 257, 520, 128, 64, 0.5, "batch_head", "bh"),
    (torch.bfloat16, 128, False, 200, 300, 64, 128, 0.5, "head", "h"),
    (torch.bfloat16, 128, True, 130, 260, 64, 64, 0.5, "batch_head", "bhi"),
]


@pytest.mark.parametrize("dtype,d,causal,nq,nk,bq,bk,density,layout,db", SPARSE_BIAS_CASES)
def test_block_bitmap_with_bias_tensor(dtype, d, causal, nq, nk, bq, bk, density, layout, db):
    # a block bitmap and a bias tensor together: forward (plain and split), backward and
    # dbias against the oracle, which applies both
    B, H = 2, 2
    seed = 23001 + nq + 5 * nk + bq + bk + d
    q, k, v, do = (normal((B, H, n, d), dtype, seed + i) for i, n in enumerate((nq, nk, nk, nq)))
    nbq, nbk = -(-nq // bq), -(-nk // bk)
    shape = {"shared": (nbq, nbk), "head": (H, nbq, nbk), "batch_head": (B, H, nbq, nbk)}[layout]
    bm = (np.random.default_rng(seed + 5).random(shape) < density).astype(np.uint8)
    bias = bias_tensor((1, H, nq, nk), seed + 6, 2.0, 0.05)
    scale = 1.0 / math.sqrt(d)
    qd, kd, vd, dod, bd = (t.to(DEV) for t in (q, k, v, do, bias))
    kw = dict(causal=causal, scale=scale, bias=bd,
              block_mask=(torch.from_numpy(bm).to(DEV), bq, bk))
    o, lse = fa.fa_fwd(qd, kd, vd, **kw)
    o2, lse2 = fa.fa_fwd_split(qd, kd, vd, n_split=3, **kw)
    dbias = None
    axes = {"dense": "", "rows": "i"}.get(db, db)
    if db is not None:
        dshape = (1 if "b" in axes else B, 1 if "h" in axes else H, 1 if "i" in axes else nq, nk)
        dbias = torch.full(dshape, float("nan"), dtype=torch.float32, device=DEV)
    dq, dk, dv = fa.fa_bwd(dod, qd, kd, vd, o, lse, dbias=dbias, **kw)
    torch.cuda.synchronize()
    bn = bias.double().numpy()
    qn, kn, vn, don = np64(q), np64(k), np64(v), np64(do)
    o_ref, lse_ref = oracle.attention_forward(qn, kn, vn, scale, causal=causal, bias=bn,
                                              block_mask=(bm, bq, bk))
    what = f"bitmap+bias {layout} {nq}x{nk} {bq}x{bk} c{causal} d{d}"
    assert_fwd_close(np64(o), np64(lse), o_ref, lse_ref, dtype, what)
    assert_fwd_close(np64(o2), np64(lse2), o_ref, lse_ref, dtype, what + " split")
    *want, dref = oracle.attention_backward(qn, kn, vn, don, scale, causal=causal, bias=bn,
                                            block_mask=(bm, bq, bk), return_dbias=True)
    check((dq, dk, dv), want, ("dQ", "dK", "dV"), what)
    if db is None:
        return
    tol, masked = dbias_tol_masked(qn, kn, vn, don, scale, causal, bn, bm, bq, bk)
    g = np64(dbias)
    assert np.isfinite(g).all(), what
    if axes == "":
        assert np.all(np.abs(g - dref) <= tol), what
        assert np.all(g[masked] == 0), what
    else:
        # summed: the sum of the per-element bounds plus the float32 rounding of a sum of
        # n terms; an element whose every summand is masked is exactly zero
        red = tuple(ax for ax, c in enumerate("bhi") if c in axes)
        n_terms = int(np.prod([(B, H, nq)[ax] for ax in red]))
        ref = dref.sum(axis=red, keepdims=True)
        bound = (tol.sum(axis=red, keepdims=True)
                 + n_terms * 2.0 ** -23 * np.abs(dref).sum(axis=red, keepdims=True))
        assert g.shape == ref.shape, what
        assert np.all(np.abs(g - ref) <= bound), what
        assert np.all(g[masked.all(axis=red, keepdims=True)] == 0), what
        if "b" in axes or "h" in axes:
            # deterministic: a second call gives the same bits
            dbias2 = torch.full(dshape, float("nan"), dtype=torch.float32, device=DEV)
            fa.fa_bwd(dod, qd, kd, vd, o, lse, dbias=dbias2, **kw)
            torch.cuda.synchronize()
            assert torch.equal(dbias, dbias2), what


def dbias_tol_masked(q, k, v, do, scale, causal, bias, bm, bq, bk):
    """dbias_tol (module docstring) with the block bitmap applied too."""
    B, H, nq, _ = q.shape
    nk = k.shape[2]
    tol = np.empty((B, H, nq, nk))
    masked = np.empty((B, H, nq, nk), dtype=bool)
    for b in range(B):
        for h in range(H):
            p = oracle.attention_probabilities(q, k, scale, b, h, causal, bias=bias,
                                               block_mask=(bm, bq, bk))
            a = (np.abs(do[b, h]) * (p @ np.abs(v[b, h]))).sum(axis=1)
            tol[b, h] = p * (2.0 ** -8 * a[:, None] + 1e-3) + 1e-6
            masked[b, h] = p == 0
    return tol, masked
