"""Pins of the oracle's bias-tensor path (``bias=`` and ``return_dbias=`` of
``oracle.attention_forward`` / ``attention_backward``). CPU only.

Source: scifaro.com related-papers page for FlashMask (arXiv 2410.01359), the abstract
on attention with bias: an additive bias matrix on the query-key scores. Readings: the
bias is added after scaling; -inf entries mask; its gradient is dS.

Pins: 50-digit brute force (scalar loops, mpmath) for the forward and central
differences of the loss for dbias; closed forms (a per-row constant bias shifts LSE
only; a bias of log 2 on one key equals that key taken twice); a -inf bias equals the
causal mask; torch autograd of torch's float64 attention with a float mask; the
generated-slope path the library already has.
"""

import math

import mpmath
import numpy as np
import pytest
import torch

import oracle

mpmath.mp.dps = 50


def rnd(shape, seed, scale=1.0):
    return np.random.default_rng(seed).standard_normal(shape) * scale


def mp_forward(q, k, v, scale, bias, causal):
    """O, LSE of one head by scalar loops in 50 digits; bias[i][j] may be -inf."""
    n_q, n_k, d = len(q), len(k), len(q[0])
    off = n_k - n_q
    O, L = [], []
    for i in range(n_q):
        sc = {}
        for j in range(n_k):
            if causal and j > i + off:
                continue
            bij = bias[i][j]
            if bij == -math.inf:
                continue
            acc = mpmath.mpf(0)
            for c in range(d):
                acc += mpmath.mpf(q[i][c]) * mpmath.mpf(k[j][c])
            sc[j] = acc * mpmath.mpf(scale) + mpmath.mpf(bij)
        if not sc:
            O.append([mpmath.mpf(0)] * d)
            L.append(-mpmath.inf)
            continue
        z = mpmath.fsum(mpmath.exp(x) for x in sc.values())
        O.append([mpmath.fsum(mpmath.exp(x) * mpmath.mpf(v[j][c]) for j, x in sc.items()) / z
                  for c in range(d)])
        L.append(mpmath.log(z))
    return O, L


def _bias(n_q, n_k, seed, frac_inf=0.0, empty_row=None):
    b = rnd((n_q, n_k), seed)
    if frac_inf:
        b[np.random.default_rng(seed + 1).random((n_q, n_k)) < frac_inf] = -np.inf
    if empty_row is not None:
        b[empty_row] = -np.inf
    return b


@pytest.mark.parametrize("causal,n_q,n_k,frac_inf", [
    (False, 5, 7, 0.0), (True, 6, 6, 0.2), (True, 4, 9, 0.3), (False, 7, 3, 0.25),
])
def test_forward_with_bias_matches_multiprecision_brute_force(causal, n_q, n_k, frac_inf):
    d = 4
    q, k, v = rnd((n_q, d), 1), rnd((n_k, d), 2), rnd((n_k, d), 3)
    b = _bias(n_q, n_k, 4, frac_inf, empty_row=1)
    o, lse = oracle.attention_forward(q[None, None], k[None, None], v[None, None], 0.6,
                                      causal=causal, bias=b[None, None])
    O, L = mp_forward(q, k, v, 0.6, b.tolist(), causal)
    for i in range(n_q):
        if L[i] == -mpmath.inf:
            assert lse[0, 0, i] == -np.inf and np.all(o[0, 0, i] == 0)
            continue
        assert abs(lse[0, 0, i] - float(L[i])) <= 1e-13
        assert np.max(np.abs(o[0, 0, i] - np.array([float(x) for x in O[i]]))) <= 1e-13


@pytest.mark.parametrize("causal", [False, True])
def test_dbias_matches_multiprecision_finite_differences(causal):
    n_q, n_k, d = 4, 5, 3
    q, k, v, do = rnd((n_q, d), 11), rnd((n_k, d), 12), rnd((n_k, d), 13), rnd((n_q, d), 14)
    b = _bias(n_q, n_k, 15, 0.15)
    *_, db = oracle.attention_backward(q[None, None], k[None, None], v[None, None],
                                       do[None, None], 0.8, causal=causal, bias=b[None, None],
                                       return_dbias=True)
    hstep = mpmath.mpf("1e-20")

    def loss(bb):
        O, _ = mp_forward(q, k, v, 0.8, bb, causal)
        return mpmath.fsum(O[i][c] * mpmath.mpf(do[i][c]) for i in range(n_q) for c in range(d))

    for i in range(n_q):
        for j in range(n_k):
            if b[i, j] == -np.inf or (causal and j > i + n_k - n_q):
                assert db[0, 0, i, j] == 0  # masked: no gradient
                continue
            bp = [[mpmath.mpf(x) for x in row] for row in b.tolist()]
            bm = [list(row) for row in bp]
            bp[i][j] += hstep
            bm[i][j] -= hstep
            fd = float((loss(bp) - loss(bm)) / (2 * hstep))
            assert abs(fd - db[0, 0, i, j]) <= 1e-12, (i, j, fd, db[0, 0, i, j])


def test_row_constant_bias_shifts_lse_only():
    # softmax is invariant to a per-row constant: O unchanged, LSE_i + c_i
    B, H, n_q, n_k, d = 1, 2, 9, 11, 8
    q, k, v = (rnd((B, H, n, d), 20 + i) for i, n in enumerate((n_q, n_k, n_k)))
    c = rnd((1, H, n_q, 1), 24, 5.0)
    o0, l0 = oracle.attention_forward(q, k, v, 0.4, causal=True)
    o1, l1 = oracle.attention_forward(q, k, v, 0.4, causal=True, bias=c)
    assert np.allclose(o1, o0, atol=1e-13, rtol=0)
    assert np.allclose(l1, l0 + c[..., 0], atol=1e-12, rtol=0)


def test_log2_bias_equals_the_key_taken_twice():
    # exp(s + log 2) = 2 exp(s): key j with bias log 2 counts like two copies of key j
    n_q, n_k, d, j = 6, 7, 5, 3
    q, k, v = rnd((n_q, d), 30), rnd((n_k, d), 31), rnd((n_k, d), 32)
    b = np.zeros((n_q, n_k))
    b[:, j] = math.log(2.0)
    o, lse = oracle.attention_forward(q[None, None], k[None, None], v[None, None], 0.5,
                                      bias=b[None, None])
    k2, v2 = np.vstack([k, k[j:j + 1]]), np.vstack([v, v[j:j + 1]])
    o2, lse2 = oracle.attention_forward(q[None, None], k2[None, None], v2[None, None], 0.5)
    assert np.allclose(o, o2, atol=1e-13, rtol=0) and np.allclose(lse, lse2, atol=1e-13, rtol=0)


def test_neg_inf_bias_equals_the_causal_mask():
    B, H, n, d = 1, 2, 10, 6
    q, k, v, do = (rnd((B, H, n, d), 40 + i) for i in range(4))
    i, jj = np.arange(n)[:, None], np.arange(n)[None, :]
    b = np.where(jj <= i, 0.0, -np.inf)[None, None]
    ref = oracle.attention_forward(q, k, v, 0.7, causal=True)
    got = oracle.attention_forward(q, k, v, 0.7, bias=b)
    for x, y in zip(ref, got):
        assert np.array_equal(x, y)
    gref = oracle.attention_backward(q, k, v, do, 0.7, causal=True)
    *g, db = oracle.attention_backward(q, k, v, do, 0.7, bias=b, return_dbias=True)
    for x, y in zip(gref, g):
        assert np.allclose(x, y, atol=1e-14, rtol=0)
    assert np.all(db[..., jj > i] == 0)


def test_tensor_bias_equals_generated_slope_bias():
    # the bias slope |i - j| given as a tensor: same outputs and gradients; and
    # sum_ij dbias |i - j| is the slope gradient of the generated path
    B, H, n_q, n_k, d = 2, 3, 8, 12, 4
    q, k, v, do = (rnd((B, H, n, d), 50 + i) for i, n in enumerate((n_q, n_k, n_k, n_q)))
    slopes = np.array([-0.3, 0.1, 0.25])
    dist = np.abs(np.arange(n_q)[:, None] - np.arange(n_k)[None, :]).astype(np.float64)
    bt = (slopes[:, None, None] * dist)[None]
    for x, y in zip(oracle.attention_forward(q, k, v, 0.5, causal=True, bias_slopes=slopes),
                    oracle.attention_forward(q, k, v, 0.5, causal=True, bias=bt)):
        assert np.allclose(x, y, atol=1e-13, rtol=0)
    *g1, dsl = oracle.attention_backward(q, k, v, do, 0.5, causal=True, bias_slopes=slopes,
                                         return_dslopes=True)
    *g2, db = oracle.attention_backward(q, k, v, do, 0.5, causal=True, bias=bt,
                                        return_dbias=True)
    for x, y in zip(g1, g2):
        assert np.allclose(x, y, atol=1e-13, rtol=0)
    assert np.allclose((db * dist).sum(axis=(0, 2, 3)), dsl, atol=1e-12, rtol=0)


def test_dbias_rows_sum_to_zero():
    # sum_j P_ij (dP_ij - D_i) = D_i - D_i sum_j P_ij = 0 for every non-empty row
    B, H, n_q, n_k, d = 2, 2, 9, 13, 8
    q, k, v, do = (rnd((B, H, n, d), 60 + i) for i, n in enumerate((n_q, n_k, n_k, n_q)))
    b = rnd((B, H, n_q, n_k), 65)
    *_, db = oracle.attention_backward(q, k, v, do, 0.3, causal=True, bias=b,
                                       return_dbias=True)
    assert np.allclose(db.sum(axis=3), 0, atol=1e-13)
    assert np.abs(db).max() > 1e-3


def test_dbias_against_torch_autograd_with_broadcast_bias():
    # torch's float64 attention with a float mask; a bias broadcast over batches and rows
    # (shape [1, H, 1, N_k]): its gradient is dbias summed over the broadcast axes
    B, H, n_q, n_k, d = 2, 3, 7, 10, 8
    q, k, v, do = (rnd((B, H, n, d), 70 + i) for i, n in enumerate((n_q, n_k, n_k, n_q)))
    b = rnd((1, H, 1, n_k), 75)
    tb = torch.tensor(b, requires_grad=True)
    tq, tk, tv = (torch.tensor(x, requires_grad=True) for x in (q, k, v))
    out = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, attn_mask=tb, scale=0.45)
    (out * torch.tensor(do)).sum().backward()
    o, _ = oracle.attention_forward(q, k, v, 0.45, bias=b)
    assert np.allclose(o, out.detach().numpy(), atol=1e-13, rtol=0)
    dq, dk, dv, db = oracle.attention_backward(q, k, v, do, 0.45, bias=b, return_dbias=True)
    for x, t in ((dq, tq), (dk, tk), (dv, tv)):
        assert np.allclose(x, t.grad.numpy(), atol=1e-12, rtol=0)
    assert np.allclose(db.sum(axis=(0, 2), keepdims=True), tb.grad.numpy(), atol=1e-12, rtol=0)


@pytest.mark.parametrize("br,bc,causal", [(4, 3, False), (5, 8, True), (16, 16, True)])
def test_tiled_online_with_bias_equals_two_pass(br, bc, causal):
    B, H, n_q, n_k, d = 1, 2, 19, 21, 8
    q, k, v = (rnd((B, H, n, d), 80 + i) for i, n in enumerate((n_q, n_k, n_k)))
    b = rnd((B, H, n_q, n_k), 84, 3.0)
    b[0, 1, 4] = -np.inf  # an empty row
    b[0, 0, :, 5:9] = -np.inf
    ref = oracle.attention_forward(q, k, v, 0.6, causal=causal, bias=b)
    got = oracle.tiled_online_forward(q, k, v, 0.6, br, bc, causal=causal, bias=b)
    assert np.allclose(got[0], ref[0], atol=1e-13, rtol=0)
    assert np.array_equal(np.isneginf(got[1]), np.isneginf(ref[1]))
    fin = np.isfinite(ref[1])
    assert np.allclose(got[1][fin], ref[1][fin], atol=1e-13, rtol=0)
