"""Pins for the CPU oracle (no GPU).

The oracle is checked against things other than itself:
* brute force in 50-digit multiprecision arithmetic (scalar loops, mpmath);
* gradients by central finite differences of that multiprecision forward;
* torch's CPU float64 reference routines (scaled_dot_product_attention, autograd);
* closed forms (single key, two keys, uniform scores, bias-only geometric sums);
* invariants (rows of P sum to 1, constant V, permutation of keys, masked keys
  equal removed keys, sum of dK is zero, sum of dV equals sum of dO);
* the tiled online recurrence of the blog's "Algoritma Flash Attention" section
  against the two-pass oracle;
* brute-force recounting for the row-block summary and tile classes.
"""

import math

import mpmath
import numpy as np
import pytest
import torch

import oracle
from oracle import attention as A
from synth import key_ranges

mpmath.mp.dps = 50


def rnd(shape, seed, scale=1.0):
    return np.random.default_rng(seed).standard_normal(shape) * scale


# --------------------------------------------------------------------------
# brute force in multiprecision: scalar loops written from the definition
# softmax(scale * q.k + bias) over the visible keys, then the weighted sum of v.
# --------------------------------------------------------------------------

def mp_forward_row(qi, K, V, scale, i, n_q, causal, slope, ks, ke, blocks=None):
    n_k, d = len(K), len(K[0])
    vis = []
    for j in range(n_k):
        ok = True
        if causal and j > i + n_k - n_q:
            ok = False
        if ks is not None and not (ks[i] <= j < ke[i]):
            ok = False
        if blocks is not None:
            bm, bq, bk = blocks
            if bm[i // bq][j // bk] == 0:
                ok = False
        if ok:
            vis.append(j)
    if not vis:
        return [mpmath.mpf(0)] * d, -mpmath.inf
    sc = {}
    for j in vis:
        acc = mpmath.mpf(0)
        for c in range(d):
            acc += mpmath.mpf(qi[c]) * mpmath.mpf(K[j][c])
        acc *= mpmath.mpf(scale)
        if slope is not None:
            acc += mpmath.mpf(slope) * abs(i - j)
        sc[j] = acc
    z = mpmath.fsum(mpmath.exp(sc[j]) for j in vis)
    out = []
    for c in range(d):
        out.append(mpmath.fsum(mpmath.exp(sc[j]) * mpmath.mpf(V[j][c]) for j in vis) / z)
    return out, mpmath.log(z)


def mp_forward(q, k, v, scale, causal=False, slope=None, ks=None, ke=None, blocks=None):
    n_q, n_k = q.shape[0], k.shape[0]
    O, L = [], []
    for i in range(n_q):
        o, l = mp_forward_row(q[i].tolist(), k.tolist(), v.tolist(), scale, i, n_q, causal,
                              slope, ks, ke, blocks)
        O.append(o)
        L.append(l)
    return O, L


CASES = [
    dict(n_q=5, n_k=5, d=3, causal=False),
    dict(n_q=6, n_k=6, d=4, causal=True),
    dict(n_q=3, n_k=7, d=2, causal=True),      # bottom-right alignment, N_q < N_k
    dict(n_q=7, n_k=4, d=3, causal=True),      # N_q > N_k: first rows see no key
    dict(n_q=6, n_k=8, d=3, causal=False, slope=-0.3),
    dict(n_q=6, n_k=6, d=2, causal=False, ranges=([0, 2, 1, 4, 3, 0], [3, 5, 1, 6, 9, -2])),
    dict(n_q=5, n_k=6, d=3, causal=True, slope=0.25, ranges=([-3, 1, 0, 2, 5], [2, 6, 4, 3, 6])),
    dict(n_q=1, n_k=1, d=4, causal=False),
]


def _case_arrays(c, seed):
    q = rnd((c["n_q"], c["d"]), seed)
    k = rnd((c["n_k"], c["d"]), seed + 1)
    v = rnd((c["n_k"], c["d"]), seed + 2)
    ks = ke = None
    if "ranges" in c:
        ks = np.array(c["ranges"][0], dtype=np.int32)
        ke = np.array(c["ranges"][1], dtype=np.int32)
    return q, k, v, ks, ke


@pytest.mark.parametrize("ci", range(len(CASES)))
def test_forward_matches_multiprecision_brute_force(ci):
    c = CASES[ci]
    q, k, v, ks, ke = _case_arrays(c, 100 + ci)
    scale = 1.0 / math.sqrt(c["d"]) * 1.3
    slope = c.get("slope")
    o, lse = oracle.attention_forward(q[None, None], k[None, None], v[None, None], scale,
                                      causal=c["causal"], bias_slopes=slope,
                                      key_start=ks, key_end=ke)
    O, L = mp_forward(q, k, v, scale, c["causal"], slope,
                      None if ks is None else ks.tolist(), None if ke is None else ke.tolist())
    for i in range(c["n_q"]):
        if L[i] == -mpmath.inf:
            assert lse[0, 0, i] == -np.inf
            assert np.all(o[0, 0, i] == 0.0)
            continue
        assert abs(float(L[i]) - lse[0, 0, i]) <= 1e-12
        for cc in range(c["d"]):
            assert abs(float(O[i][cc]) - o[0, 0, i, cc]) <= 1e-12


def _mp_loss(q, k, v, do, scale, causal, slope, ks, ke):
    O, _ = mp_forward(q, k, v, scale, causal, slope, ks, ke)
    tot = mpmath.mpf(0)
    for i in range(len(O)):
        for c in range(len(O[0])):
            tot += O[i][c] * mpmath.mpf(do[i][c])
    return tot


@pytest.mark.parametrize("ci", [0, 1, 2, 4, 6])
def test_backward_matches_multiprecision_finite_differences(ci):
    c = CASES[ci]
    q, k, v, ks, ke = _case_arrays(c, 300 + ci)
    do = rnd((c["n_q"], c["d"]), 400 + ci)
    scale = 0.7
    slope = c.get("slope")
    ksl = None if ks is None else ks.tolist()
    kel = None if ke is None else ke.tolist()
    dq, dk, dv = oracle.attention_backward(q[None, None], k[None, None], v[None, None],
                                           do[None, None], scale, causal=c["causal"],
                                           bias_slopes=slope, key_start=ks, key_end=ke)
    hstep = mpmath.mpf("1e-20")
    for name, arr, grad in (("q", q, dq), ("k", k, dk), ("v", v, dv)):
        for idx in np.ndindex(arr.shape):
            plus = [x.tolist() for x in (q, k, v)]
            minus = [x.tolist() for x in (q, k, v)]
            which = "qkv".index(name)
            plus[which][idx[0]][idx[1]] = mpmath.mpf(arr[idx]) + hstep
            minus[which][idx[0]][idx[1]] = mpmath.mpf(arr[idx]) - hstep
            fp = _mp_loss(np.array(plus[0], dtype=object), np.array(plus[1], dtype=object),
                          np.array(plus[2], dtype=object), do, scale, c["causal"], slope, ksl, kel)
            fm = _mp_loss(np.array(minus[0], dtype=object), np.array(minus[1], dtype=object),
                          np.array(minus[2], dtype=object), do, scale, c["causal"], slope, ksl,
                          kel)
            fd = float((fp - fm) / (2 * hstep))
            assert abs(fd - grad[0, 0][idx]) <= 1e-10, (name, idx, fd, grad[0, 0][idx])


@pytest.mark.parametrize("ci", [4, 6])
def test_slope_gradient_matches_multiprecision_finite_differences(ci):
    # dL/dslope = sum dS |i - j|, against a central difference of the 50-digit forward
    c = CASES[ci]
    q, k, v, ks, ke = _case_arrays(c, 500 + ci)
    do = rnd((c["n_q"], c["d"]), 600 + ci)
    scale = 0.7
    slope = c["slope"]
    ksl = None if ks is None else ks.tolist()
    kel = None if ke is None else ke.tolist()
    *_, ds = oracle.attention_backward(q[None, None], k[None, None], v[None, None],
                                       do[None, None], scale, causal=c["causal"],
                                       bias_slopes=slope, key_start=ks, key_end=ke,
                                       return_dslopes=True)
    hstep = mpmath.mpf("1e-20")
    fp = _mp_loss(q, k, v, do, scale, c["causal"], mpmath.mpf(slope) + hstep, ksl, kel)
    fm = _mp_loss(q, k, v, do, scale, c["causal"], mpmath.mpf(slope) - hstep, ksl, kel)
    fd = float((fp - fm) / (2 * hstep))
    assert ds.shape == (1,) and abs(fd - ds[0]) <= 1e-10, (fd, ds)


def test_slope_gradient_per_head_and_shared_against_torch_autograd():
    # per-head slopes: one gradient each; one shared slope: the sum over heads
    B, H, n_q, n_k, d = 2, 3, 19, 23, 8
    q, k, v, do = (rnd((B, H, n, d), 700 + i) for i, n in enumerate((n_q, n_k, n_k, n_q)))
    slopes = np.array([-0.2, 0.05, 0.1])
    ts = torch.tensor(slopes, dtype=torch.float64, requires_grad=True)
    dist = (torch.arange(n_q)[:, None] - torch.arange(n_k)[None, :]).abs().double()
    allowed = torch.arange(n_k)[None, :] <= torch.arange(n_q)[:, None] + (n_k - n_q)
    bias = (ts[:, None, None] * dist).masked_fill(~allowed, float("-inf"))
    out = torch.nn.functional.scaled_dot_product_attention(
        torch.tensor(q), torch.tensor(k), torch.tensor(v), attn_mask=bias, scale=0.3)
    (out * torch.tensor(do)).sum().backward()
    *_, ds = oracle.attention_backward(q, k, v, do, 0.3, causal=True, bias_slopes=slopes,
                                       return_dslopes=True)
    assert np.allclose(ds, ts.grad.numpy(), atol=1e-12, rtol=0)
    *_, ds1 = oracle.attention_backward(q, k, v, do, 0.3, causal=True, bias_slopes=[0.07],
                                        return_dslopes=True)
    t1 = torch.tensor(0.07, dtype=torch.float64, requires_grad=True)
    out1 = torch.nn.functional.scaled_dot_product_attention(
        torch.tensor(q), torch.tensor(k), torch.tensor(v),
        attn_mask=(t1 * dist).masked_fill(~allowed, float("-inf")), scale=0.3)
    (out1 * torch.tensor(do)).sum().backward()
    assert ds1.shape == (1,) and abs(ds1[0] - float(t1.grad)) <= 1e-12


# --------------------------------------------------------------------------
# torch's CPU float64 reference routines (an independent library path)
# --------------------------------------------------------------------------

def _torch_ref(q, k, v, scale, causal, slope, ks, ke):
    n_q, n_k = q.shape[2], k.shape[2]
    i = torch.arange(n_q)[:, None]
    j = torch.arange(n_k)[None, :]
    allowed = torch.ones(n_q, n_k, dtype=torch.bool)
    if causal:
        allowed &= j <= i + (n_k - n_q)
    if ks is not None:
        allowed &= (j >= torch.as_tensor(ks, dtype=torch.int64)[:, None]) & \
                   (j < torch.as_tensor(ke, dtype=torch.int64)[:, None])
    bias = torch.zeros(n_q, n_k, dtype=torch.float64)
    if slope is not None:
        bias = slope * (i - j).abs().double()
    add = bias.masked_fill(~allowed, float("-inf"))
    tq, tk, tv = (torch.tensor(x, dtype=torch.float64, requires_grad=True) for x in (q, k, v))
    out = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, attn_mask=add, scale=scale)
    return out, (tq, tk, tv), allowed


@pytest.mark.parametrize("causal,slope,masked,n_q,n_k", [
    (False, None, False, 37, 37),
    (True, None, False, 40, 40),
    (True, None, False, 23, 50),
    (False, -0.05, False, 33, 29),
    (False, -0.1 / 64, True, 64, 64),
    (True, 0.02, True, 31, 31),
])
def test_against_torch_float64_reference(causal, slope, masked, n_q, n_k):
    B, H, d = 2, 3, 16
    q = rnd((B, H, n_q, d), 1)
    k = rnd((B, H, n_k, d), 2)
    v = rnd((B, H, n_k, d), 3)
    do = rnd((B, H, n_q, d), 4)
    ks = ke = None
    if masked:
        s_, e_ = key_ranges(n_q, n_k, seed=77, block=8, width=n_k // 2, jitter=4)
        ks, ke = s_.numpy(), e_.numpy()
    scale = 1.0 / math.sqrt(d)
    out, (tq, tk, tv), allowed = _torch_ref(q, k, v, scale, causal, slope, ks, ke)
    rows_ok = allowed.any(dim=1)
    o, lse = oracle.attention_forward(q, k, v, scale, causal, slope, ks, ke)
    # torch gives NaN on rows with no visible key; the oracle's reading there is O=0
    assert np.allclose(o[:, :, rows_ok.numpy()], out.detach().numpy()[:, :, rows_ok.numpy()],
                       atol=1e-13, rtol=0)
    if (~rows_ok).any():
        assert np.all(o[:, :, ~rows_ok.numpy()] == 0)
        assert np.all(lse[:, :, ~rows_ok.numpy()] == -np.inf)
    # LSE from torch's logsumexp of the same masked scores
    s_t = scale * torch.tensor(q) @ torch.tensor(k).transpose(-1, -2)
    if slope is not None:
        s_t = s_t + slope * (torch.arange(n_q)[:, None] - torch.arange(n_k)[None, :]).abs().double()
    s_t = s_t.masked_fill(~allowed, float("-inf"))
    lse_t = torch.logsumexp(s_t, dim=-1).numpy()
    assert np.allclose(lse[:, :, rows_ok.numpy()], lse_t[:, :, rows_ok.numpy()], atol=1e-12)
    if (~rows_ok).any():
        return  # torch's gradients through all-masked rows are NaN
    (out * torch.tensor(do)).sum().backward()
    dq, dk, dv = oracle.attention_backward(q, k, v, do, scale, causal, slope, ks, ke)
    assert np.allclose(dq, tq.grad.numpy(), atol=1e-12, rtol=0)
    assert np.allclose(dk, tk.grad.numpy(), atol=1e-12, rtol=0)
    assert np.allclose(dv, tv.grad.numpy(), atol=1e-12, rtol=0)


# --------------------------------------------------------------------------
# closed forms
# --------------------------------------------------------------------------

def test_single_key_returns_v():
    q, k, v = rnd((1, 2, 9, 8), 5), rnd((1, 2, 1, 8), 6), rnd((1, 2, 1, 8), 7)
    o, lse = oracle.attention_forward(q, k, v, 0.4)
    assert np.array_equal(o, np.broadcast_to(v, o.shape))
    s00 = 0.4 * (q @ np.swapaxes(k, -1, -2))[..., 0]
    assert np.allclose(lse, s00, atol=1e-14, rtol=0)


def test_two_keys_logistic():
    q, k, v = rnd((1, 1, 6, 1), 8), rnd((1, 1, 2, 1), 9), rnd((1, 1, 2, 1), 10)
    scale = 0.9
    o, lse = oracle.attention_forward(q, k, v, scale)
    s0 = scale * q[0, 0, :, 0] * k[0, 0, 0, 0]
    s1 = scale * q[0, 0, :, 0] * k[0, 0, 1, 0]
    sig = 1.0 / (1.0 + np.exp(-(s0 - s1)))
    want = sig * v[0, 0, 0, 0] + (1 - sig) * v[0, 0, 1, 0]
    assert np.allclose(o[0, 0, :, 0], want, atol=1e-14, rtol=0)
    assert np.allclose(lse[0, 0], np.logaddexp(s0, s1), atol=1e-14, rtol=0)


@pytest.mark.parametrize("causal", [False, True])
def test_uniform_scores_mean_of_visible_values(causal):
    n = 19
    q = np.zeros((1, 1, n, 4))
    k, v = rnd((1, 1, n, 4), 11), rnd((1, 1, n, 4), 12)
    o, lse = oracle.attention_forward(q, k, v, 0.5, causal=causal)
    for i in range(n):
        nvis = i + 1 if causal else n
        assert abs(lse[0, 0, i] - math.log(nvis)) <= 1e-14
        assert np.allclose(o[0, 0, i], v[0, 0, :nvis].mean(axis=0), atol=1e-14, rtol=0)


def test_bias_only_geometric_series():
    n, c = 300, 0.1 / 64
    q = np.zeros((1, 1, n, 2))
    k, v = rnd((1, 1, n, 2), 13), rnd((1, 1, n, 2), 14)
    s_, e_ = key_ranges(n, n, seed=3, block=32, width=120, jitter=16)
    ks, ke = s_.numpy(), e_.numpy()
    _, lse = oracle.attention_forward(q, k, v, 1.0, bias_slopes=-c, key_start=ks, key_end=ke)
    r = math.exp(-c)
    for i in range(n):
        a, b = max(ks[i], 0), min(ke[i], n)  # visible keys [a, b)
        tot = 0.0
        # sum_{j in [a,b)} r^{|i-j|}, split at i, each a finite geometric series
        lo_hi = min(b, i + 1)
        if a < lo_hi:  # j in [a, lo_hi): exponent i-j runs from i-lo_hi+1 .. i-a
            e0, e1 = i - lo_hi + 1, i - a
            tot += r ** e0 * (1 - r ** (e1 - e0 + 1)) / (1 - r)
        hi_lo = max(a, i + 1)
        if hi_lo < b:  # j in [hi_lo, b): exponent j-i runs from hi_lo-i .. b-1-i
            e0, e1 = hi_lo - i, b - 1 - i
            tot += r ** e0 * (1 - r ** (e1 - e0 + 1)) / (1 - r)
        assert abs(lse[0, 0, i] - math.log(tot)) <= 1e-12


def test_constant_v_gives_constant_output_and_zero_dq_dk():
    n, d = 33, 8
    q, k = rnd((1, 2, n, d), 15), rnd((1, 2, n, d), 16)
    u = rnd((d,), 17)
    v = np.broadcast_to(u, (1, 2, n, d)).copy()
    do = rnd((1, 2, n, d), 18)
    o, _ = oracle.attention_forward(q, k, v, 0.3, causal=True)
    assert np.allclose(o, np.broadcast_to(u, o.shape), atol=1e-14, rtol=0)
    dq, dk, _ = oracle.attention_backward(q, k, v, do, 0.3, causal=True)
    assert np.abs(dq).max() <= 1e-13 and np.abs(dk).max() <= 1e-13


# --------------------------------------------------------------------------
# invariants
# --------------------------------------------------------------------------

def test_probability_rows_sum_to_one():
    n = 40
    q, k = rnd((1, 1, n, 8), 19), rnd((1, 1, n, 8), 20)
    s_, e_ = key_ranges(n, n, seed=5, block=8, width=12, jitter=4)
    p = oracle.attention_probabilities(q, k, 0.5, causal=True, bias_slopes=-0.01,
                                       key_start=s_.numpy(), key_end=e_.numpy())
    vis = A.visible_mask(n, n, np.arange(n), True, s_.numpy(), e_.numpy())
    has = vis.any(axis=1)
    assert np.allclose(p[has].sum(axis=1), 1.0, atol=1e-14, rtol=0)
    assert np.all(p[~vis] == 0)
    assert np.all(p[~has] == 0)


def test_key_value_permutation_invariance():
    n_q, n_k = 17, 29
    q, k, v = rnd((2, 2, n_q, 8), 21), rnd((2, 2, n_k, 8), 22), rnd((2, 2, n_k, 8), 23)
    perm = np.random.default_rng(0).permutation(n_k)
    o1, l1 = oracle.attention_forward(q, k, v, 0.35)
    o2, l2 = oracle.attention_forward(q, k[:, :, perm], v[:, :, perm], 0.35)
    assert np.allclose(o1, o2, atol=1e-14, rtol=0) and np.allclose(l1, l2, atol=1e-14, rtol=0)


def test_masked_keys_equal_removed_keys():
    n_q, n_k = 9, 20
    q, k, v = rnd((1, 1, n_q, 4), 24), rnd((1, 1, n_k, 4), 25), rnd((1, 1, n_k, 4), 26)
    ks = np.full(n_q, 5, dtype=np.int32)
    ke = np.full(n_q, 13, dtype=np.int32)
    o1, l1 = oracle.attention_forward(q, k, v, 0.5, key_start=ks, key_end=ke)
    o2, l2 = oracle.attention_forward(q, k[:, :, 5:13], v[:, :, 5:13], 0.5)
    assert np.allclose(o1, o2, atol=1e-14, rtol=0) and np.allclose(l1, l2, atol=1e-14, rtol=0)


def test_gradient_sums():
    n = 48
    q, k, v, do = (rnd((1, 2, n, 8), s) for s in (27, 28, 29, 30))
    dq, dk, dv = oracle.attention_backward(q, k, v, do, 0.3, causal=True, bias_slopes=-0.02)
    assert np.abs(dk.sum(axis=2)).max() <= 1e-12
    assert np.allclose(dv.sum(axis=2), do.sum(axis=2), atol=1e-12, rtol=0)


# --------------------------------------------------------------------------
# the tiled online recurrence equals the two-pass definition
# --------------------------------------------------------------------------

@pytest.mark.parametrize("br,bc,causal,bias,mask", [
    (16, 16, False, False, False),
    (7, 5, True, False, False),
    (32, 13, False, True, True),
    (64, 64, True, True, True),
    (3, 50, True, False, True),
])
def test_tiled_online_equals_two_pass(br, bc, causal, bias, mask):
    n_q, n_k, d = 71, 83, 8
    q, k, v = rnd((1, 2, n_q, d), 31, 2.0), rnd((1, 2, n_k, d), 32, 2.0), rnd((1, 2, n_k, d), 33)
    ks = ke = None
    if mask:
        s_, e_ = key_ranges(n_q, n_k, seed=9, block=16, width=30, jitter=8)
        ks, ke = s_.numpy(), e_.numpy()
    slope = -0.05 if bias else None
    o1, l1 = oracle.attention_forward(q, k, v, 0.6, causal, slope, ks, ke)
    o2, l2 = oracle.tiled_online_forward(q, k, v, 0.6, br, bc, causal, slope, ks, ke)
    assert np.allclose(o1, o2, atol=1e-12, rtol=0)
    fin = np.isfinite(l1)
    assert np.array_equal(fin, np.isfinite(l2))
    assert np.allclose(l1[fin], l2[fin], atol=1e-12, rtol=0)


# --------------------------------------------------------------------------
# row-block summary and tile classes
# --------------------------------------------------------------------------

def test_row_block_summary_brute_force():
    n_q, n_k = 1000, 700
    s_, e_ = key_ranges(n_q, n_k, seed=41, block=100, width=300, jitter=50)
    ks, ke = s_.numpy().copy(), e_.numpy().copy()
    ks[5], ke[5] = -20, 900  # out-of-range values are clamped
    summ = oracle.row_block_summary(ks, ke, n_k, 64)
    for r in range(summ.shape[0]):
        lo, hi = r * 64, min(n_q, r * 64 + 64)
        st = [min(max(int(x), 0), n_k) for x in ks[lo:hi]]
        en = [min(max(int(x), 0), n_k) for x in ke[lo:hi]]
        assert tuple(summ[r]) == (min(st), max(st), min(en), max(en))


def test_tile_classes_causal_closed_form():
    # square causal, B_r = B_c: T(T-1)/2 tiles skipped, T on the diagonal partial
    for n, b in ((256, 64), (8192, 128), (2048, 128)):
        t = n // b
        cls = oracle.tile_classes(n, n, b, b, causal=True)
        assert (cls == A.SKIP).sum() == t * (t - 1) // 2
        assert (cls == A.PARTIAL).sum() == t
        assert (cls == A.FULL).sum() == t * (t - 1) // 2


def test_tile_classes_match_summary_rule_for_generator():
    n = 2048
    s_, e_ = key_ranges(n, n, seed=9009, block=128, width=n // 2, jitter=64)
    ks, ke = s_.numpy(), e_.numpy()
    cls = oracle.tile_classes(n, n, 128, 128, key_start=ks, key_end=ke)
    summ = oracle.row_block_summary(ks, ke, n, 128)
    for r in range(cls.shape[0]):
        mn_s, mx_s, mn_e, mx_e = summ[r]
        for c in range(cls.shape[1]):
            lo, hi = c * 128, (c + 1) * 128
            if hi <= mn_s or lo >= mx_e:
                want = A.SKIP
            elif mx_s <= lo and mn_e >= hi:
                want = A.FULL
            else:
                want = A.PARTIAL
            # the summary rule never skips a tile with a visible entry
            if want == A.SKIP:
                assert cls[r, c] == A.SKIP
            if cls[r, c] == A.FULL:
                assert want == A.FULL
            # for this generator (one interval width, jitter < tile) the rule is exact
            assert cls[r, c] == want


def test_half_of_tiles_skipped_for_range_mask_generator():
    n = 8192
    s_, e_ = key_ranges(n, n, seed=4009, block=128, width=n // 2, jitter=64)
    cls = oracle.tile_classes(n, n, 128, 128, key_start=s_.numpy(), key_end=e_.numpy())
    frac = (cls == A.SKIP).mean()
    assert 0.45 <= frac <= 0.55


# --------------------------------------------------------------------------
# block-sparse bitmap mask (briefgpt.xyz page for arXiv 2307.08691: the tiled method
# extends to block-sparse attention; entries of a zero block are masked)
# --------------------------------------------------------------------------

@pytest.mark.parametrize("causal,slope", [(False, None), (True, 0.2)])
def test_block_mask_matches_multiprecision_brute_force(causal, slope):
    n_q, n_k, d, bq, bk = 7, 11, 3, 2, 3
    bm = np.array([[1, 0, 1, 1], [0, 1, 0, 0], [0, 0, 0, 0], [1, 1, 0, 1]], dtype=np.uint8)
    q, k, v = rnd((n_q, d), 310), rnd((n_k, d), 311), rnd((n_k, d), 312)
    O, L = mp_forward(q, k, v, 0.7, causal, slope, blocks=(bm.tolist(), bq, bk))
    o, lse = oracle.attention_forward(q[None, None], k[None, None], v[None, None], 0.7,
                                      causal=causal, bias_slopes=slope, block_mask=(bm, bq, bk))
    for i in range(n_q):
        if L[i] == -mpmath.inf:
            assert lse[0, 0, i] == -np.inf and np.all(o[0, 0, i] == 0.0)
            continue
        assert abs(float(L[i]) - lse[0, 0, i]) < 1e-12
        assert max(abs(float(O[i][c]) - o[0, 0, i, c]) for c in range(d)) < 1e-12
    assert lse[0, 0, 4] == -np.inf and lse[0, 0, 5] == -np.inf  # block row 2 is empty


def test_block_permutation_equals_independent_problems():
    # query block r sees key block pi(r) only, with non-square blocks: each query block is
    # then an unmasked attention of its own rows over one slice of the keys
    bq, bk, nb, d = 3, 5, 4, 4
    pi = [2, 0, 3, 1]
    bm = np.zeros((nb, nb), dtype=np.uint8)
    for r, c in enumerate(pi):
        bm[r, c] = 1
    n_q, n_k = bq * nb, bk * nb
    q, k, v, do = (rnd((1, 2, n, d), 320 + i) for i, n in enumerate((n_q, n_k, n_k, n_q)))
    o, lse = oracle.attention_forward(q, k, v, 0.45, block_mask=(bm, bq, bk))
    dq, dk, dv = oracle.attention_backward(q, k, v, do, 0.45, block_mask=(bm, bq, bk))
    for r, c in enumerate(pi):
        rs, cs = slice(r * bq, (r + 1) * bq), slice(c * bk, (c + 1) * bk)
        o_r, l_r = oracle.attention_forward(q[:, :, rs], k[:, :, cs], v[:, :, cs], 0.45)
        g = oracle.attention_backward(q[:, :, rs], k[:, :, cs], v[:, :, cs], do[:, :, rs], 0.45)
        assert np.allclose(o[:, :, rs], o_r, atol=1e-14, rtol=0)
        assert np.allclose(lse[:, :, rs], l_r, atol=1e-14, rtol=0)
        assert np.allclose(dq[:, :, rs], g[0], atol=1e-13, rtol=0)
        assert np.allclose(dk[:, :, cs], g[1], atol=1e-13, rtol=0)
        assert np.allclose(dv[:, :, cs], g[2], atol=1e-13, rtol=0)


@pytest.mark.parametrize("causal", [False, True])
def test_block_mask_with_contiguous_rows_equals_key_ranges(causal):
    # a bitmap whose row r shows key blocks [a_r, b_r) is the key range [a_r bk, b_r bk)
    bq, bk, n_q, n_k, d = 4, 6, 14, 27, 3
    spans = [(0, 2), (1, 5), (3, 3), (2, 4)]
    bm = np.zeros((4, 5), dtype=np.uint8)
    for r, (lo, hi) in enumerate(spans):
        bm[r, lo:hi] = 1
    ks = np.array([spans[i // bq][0] * bk for i in range(n_q)], dtype=np.int32)
    ke = np.array([min(spans[i // bq][1] * bk, n_k) for i in range(n_q)], dtype=np.int32)
    q, k, v, do = (rnd((2, 1, n, d), 330 + i) for i, n in enumerate((n_q, n_k, n_k, n_q)))
    a = oracle.attention_forward(q, k, v, 0.6, causal=causal, block_mask=(bm, bq, bk))
    b = oracle.attention_forward(q, k, v, 0.6, causal=causal, key_start=ks, key_end=ke)
    for x, y in zip(a, b):
        assert np.array_equal(np.isinf(x), np.isinf(y))
        assert np.allclose(np.nan_to_num(x, neginf=0.0), np.nan_to_num(y, neginf=0.0), atol=1e-14, rtol=0)
    ga = oracle.attention_backward(q, k, v, do, 0.6, causal=causal, block_mask=(bm, bq, bk))
    gb = oracle.attention_backward(q, k, v, do, 0.6, causal=causal, key_start=ks, key_end=ke)
    for x, y in zip(ga, gb):
        assert np.allclose(x, y, atol=1e-13, rtol=0)


def test_block_mask_per_head_selection():
    # a [B, H, nbq, nbk] bitmap applies head by head; an all-ones bitmap changes nothing
    bq = bk = 4
    q, k, v = rnd((2, 3, 8, 3), 340), rnd((2, 3, 12, 3), 341), rnd((2, 3, 12, 3), 342)
    bm = (np.random.default_rng(343).random((2, 3, 2, 3)) < 0.6).astype(np.uint8)
    o, lse = oracle.attention_forward(q, k, v, 0.5, block_mask=(bm, bq, bk))
    for b in range(2):
        for h in range(3):
            one = lambda t: t[b:b + 1, h:h + 1]  # noqa: E731
            o1, l1 = oracle.attention_forward(one(q), one(k), one(v), 0.5, block_mask=(bm[b, h], bq, bk))
            assert np.array_equal(o[b, h], o1[0, 0]) and np.array_equal(lse[b, h], l1[0, 0])
    ones = np.ones((2, 3), dtype=np.uint8)
    o2, l2 = oracle.attention_forward(q, k, v, 0.5, block_mask=(ones, bq, bk))
    o3, l3 = oracle.attention_forward(q, k, v, 0.5)
    assert np.array_equal(o2, o3) and np.array_equal(l2, l3)


def test_tiled_online_with_block_mask_equals_two_pass():
    q, k, v = rnd((1, 2, 37, 5), 350), rnd((1, 2, 53, 5), 351), rnd((1, 2, 53, 5), 352)
    bm = (np.random.default_rng(353).random((2, 10, 11)) < 0.5).astype(np.uint8)
    o1, l1 = oracle.attention_forward(q, k, v, 0.4, causal=True, block_mask=(bm, 4, 5))
    o2, l2 = oracle.tiled_online_forward(q, k, v, 0.4, 8, 10, causal=True, block_mask=(bm, 4, 5))
    assert np.array_equal(np.isinf(l1), np.isinf(l2))
    assert np.allclose(o1, o2, atol=1e-13, rtol=0)
    fin = np.isfinite(l1)
    assert np.allclose(l1[fin], l2[fin], atol=1e-13, rtol=0)


def test_tile_classes_of_a_tile_aligned_bitmap():
    # tiles that coincide with bitmap blocks are SKIP where the byte is 0, else FULL
    bm = (np.random.default_rng(360).random((5, 7)) < 0.5).astype(np.uint8)
    cls = oracle.tile_classes(5 * 8, 7 * 16, 8, 16, blocks=(bm, 8, 16))
    assert np.array_equal(cls, np.where(bm != 0, A.FULL, A.SKIP))
