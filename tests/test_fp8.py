"""GPU parity of the FP8 path: quantiser (bit-exact codes and amaxes against the oracle)
and forward (against the float64 oracle on the same quantised operands).

Source of the method: marketmaker.cc blog on Flash Attention, section "FA3: Mekanika
hopper", item 3.

Forward tolerance, derived from the arithmetic: the kernel computes S on the E4M3 codes
with float32 accumulation (the fp8 MFMA's sum was within 2^-12 of sum |a b| in a probe on
random codes; 2^-10 is used), applies the block scales, and rounds each probability
(relative to the running max, so at most 2^8 and at least the true value over the true
row max) to E4M3 before P V; the row sum uses the unrounded values. A normal E4M3 value is
within 2^-4 relative; one below E4M3's normal range (< 2^-6) within 2^-10 absolute, and
the row sum in the same units is at least the oracle's l_rel = sum_j exp(s_ij - max_j s_ij).
So, per element (i, c), with p the oracle's probabilities and ds_i the S error bound:
    |dO_ic| <= (2^-4 + 2 ds_i) (P |Vh|)_ic + 2^-10 sum_{j: p_rel_ij < 2^-6} |Vh_jc| / l_rel_i
               + 2^-8 |O_ic| (output rounding) + 1e-4,
    ds_i = 2^-10 * scale / div * max_j (|qh_i| . |kh_j|),   |dLSE_i| <= ds_i + 1e-5 |LSE_i|.
"""

import math

import numpy as np
import pytest
import torch

import oracle
from oracle import fp8 as F
from synth import normal, random_signs, with_outliers, WORKLOADS, qkv_inputs
from tests.util import np64, sample_rows

pytestmark = pytest.mark.gpu

fa = pytest.importorskip("exact_io_aware_flash_amd")
DEV = "cuda:0"


# ---- layouts (fa.h) ---------------------------------------------------------------------
def k_swz(d, r):
    return (r >> 1) & 7 if d == 128 else (r >> 2) & 3


def v_pos(k):
    return 16 * (k >> 5) + 32 * ((k >> 2) & 1) + 4 * ((k & 31) >> 3) + (k & 3)


def unpack(x8, layout):
    """Codes [B, H, Np, d] (row-major) from the library's byte order."""
    x8 = x8.cpu().numpy()
    B, H, n_p, d = x8.shape
    if layout == fa.FA_FP8_Q:
        return x8
    tiles = x8.reshape(B, H, n_p // 64, 64 * d)
    out = np.empty((B, H, n_p // 64, 64, d), dtype=np.uint8)
    r = np.arange(64)[:, None]
    e = np.arange(d)[None, :]
    if layout == fa.FA_FP8_K:
        idx = r * d + 16 * ((e // 16) ^ np.vectorize(lambda x: k_swz(d, x))(r)) + e % 16
    else:
        p = np.vectorize(v_pos)(r)
        idx = e * 64 + 16 * ((p >> 4) ^ ((e >> 2) & 3)) + (p & 15)
    out[...] = tiles[..., idx]
    return out.reshape(B, H, n_p, d)


def test_layout_maps_are_permutations():
    for d in (64, 128):
        r = np.arange(64)[:, None]
        e = np.arange(d)[None, :]
        kidx = r * d + 16 * ((e // 16) ^ np.vectorize(lambda x: k_swz(d, x))(r)) + e % 16
        p = np.vectorize(v_pos)(r)
        vidx = e * 64 + 16 * ((p >> 4) ^ ((e >> 2) & 3)) + (p & 15)
        for idx in (kidx, vidx):
            assert np.array_equal(np.sort(idx.ravel()), np.arange(64 * d))


# ---- quantiser --------------------------------------------------------------------------
QCASES = [
    # dtype, d, N, layout, rotate
    (torch.bfloat16, 128, 300, "Q", True),
    (torch.bfloat16, 128, 300, "K", True),
    (torch.bfloat16, 128, 300, "V", False),
    (torch.float16, 64, 150, "Q", False),
    (torch.float16, 64, 150, "K", True),
    (torch.float16, 64, 150, "V", False),
    (torch.bfloat16, 64, 1, "K", False),
    (torch.bfloat16, 128, 64, "V", False),
    (torch.float16, 128, 777, "Q", True),
]


@pytest.mark.parametrize("dtype,d,n,layout,rot", QCASES)
def test_quantiser_codes_bit_exact(dtype, d, n, layout, rot):
    B, H = 2, 3
    x = with_outliers((B, H, n, d), dtype, 500 + n + d, 0.01, 10.0)
    s = random_signs(d, 77) if rot else None
    lay = {"Q": fa.FA_FP8_Q, "K": fa.FA_FP8_K, "V": fa.FA_FP8_V}[layout]
    x8, amax = fa.fa_fp8_quantize(x.to(DEV), lay, s)
    torch.cuda.synchronize()
    codes, amax_ref, _ = F.quantize_v(np64(x)) if layout == "V" else F.quantize(np64(x), s)
    got = unpack(x8, lay)
    assert np.array_equal(amax.cpu().numpy(), amax_ref), "block amax"
    bad = np.argwhere(got != codes)
    assert bad.size == 0, f"{len(bad)} codes differ, first at {bad[:3].tolist()}"


def test_quantiser_rejects_bad_arguments():
    x = normal((1, 1, 64, 64), torch.bfloat16, 1).to(DEV)
    with pytest.raises(fa.FaError):
        fa.fa_fp8_quantize(x, fa.FA_FP8_V, random_signs(64, 1))  # V is never rotated
    with pytest.raises(fa.FaError):
        fa.fa_fp8_quantize(x, fa.FA_FP8_Q, [0.5] * 64)  # signs must be +-1
    with pytest.raises(fa.FaError):
        fa.fa_fp8_quantize(x, 7)


# ---- forward ----------------------------------------------------------------------------
def reference(q, k, v, scale, causal, signs):
    qh, kh, vh, div = F.fp8_attention_operands(np64(q), np64(k), np64(v), signs)
    o, lse = oracle.attention_forward(qh, kh, vh, scale / div, causal=causal)
    return qh, kh, vh, div, o, lse


def check_fp8(o, lse, qh, kh, vh, div, o_ref, lse_ref, scale, causal, what, rows=None):
    """Kernel O / LSE of the given rows against the oracle on the same quantised operands,
    within the bound derived in the module docstring (per element)."""
    o, lse = np64(o), np64(lse)
    B, H, n_q, d = qh.shape
    rows = np.arange(n_q) if rows is None else np.asarray(rows)
    for b in range(B):
        for h in range(H):
            ref, lref = o_ref[b, h, rows], lse_ref[b, h, rows]
            empty = ~np.isfinite(lref)
            assert np.all(o[b, h, rows][empty] == 0) and np.all(np.isneginf(lse[b, h, rows][empty]))
            s_rows = oracle.scores(qh[b, h, rows], kh[b, h], scale / div, rows, n_q, causal)
            m = np.where(empty, 0.0, s_rows.max(axis=1))
            p_rel = np.exp(s_rows - m[:, None])        # 1 at the row max
            l_rel = np.maximum(p_rel.sum(axis=1), 1.0)
            p = p_rel / l_rel[:, None]
            av = np.abs(vh[b, h])
            # S error of the fp8 products (natural-log units), per row
            ds = 2.0 ** -10 * scale / div * (np.abs(qh[b, h, rows]) @ np.abs(kh[b, h]).T).max(axis=1)
            small = (p_rel < 2.0 ** -6).astype(np.float64)
            tol = ((2.0 ** -4 + 2 * ds[:, None]) * (p @ av)
                   + 2.0 ** -10 * (small @ av) / l_rel[:, None]
                   + 2.0 ** -8 * np.abs(ref) + 1e-4)
            err = np.abs(o[b, h, rows] - ref)
            worst = np.unravel_index(np.argmax(err - tol), err.shape)
            assert np.all(err <= tol), (f"{what} b{b} h{h}: |dO| {err[worst]:.3e} > "
                                        f"{tol[worst]:.3e} at row {rows[worst[0]]}")
            fin = ~empty
            lerr = np.abs(lse[b, h, rows][fin] - lref[fin])
            ltol = ds[fin] + 1e-5 * np.abs(lref[fin])
            assert np.all(lerr <= ltol), f"{what} b{b} h{h}: |dLSE| {lerr.max():.3e}"


FCASES = [
    # dtype, d, causal, nq, nk, rotate
    (torch.bfloat16, 128, True, 300, 300, True),
    (torch.bfloat16, 128, False, 200, 520, False),
    (torch.float16, 64, True, 333, 700, True),
    (torch.float16, 64, False, 64, 64, False),
    (torch.bfloat16, 128, True, 1, 1000, True),
    (torch.bfloat16, 64, True, 520, 130, False),
]


@pytest.mark.parametrize("dtype,d,causal,nq,nk,rot", FCASES)
def test_fp8_forward_matches_oracle(dtype, d, causal, nq, nk, rot):
    B, H = 2, 2
    seed = 600 + nq + nk + d
    q, k, v = (normal((B, H, n, d), dtype, seed + i) for i, n in enumerate((nq, nk, nk)))
    s = random_signs(d, seed + 9) if rot else None
    scale = 1.0 / math.sqrt(d)
    o, lse = fa.fa_attention_fp8(q.to(DEV), k.to(DEV), v.to(DEV), causal=causal, scale=scale,
                                 signs=s)
    torch.cuda.synchronize()
    assert o.dtype == dtype
    qh, kh, vh, div, o_ref, lse_ref = reference(q, k, v, scale, causal, s)
    check_fp8(o, lse, qh, kh, vh, div, o_ref, lse_ref, scale, causal,
              f"fp8 {dtype} d{d} c{causal} {nq}x{nk} rot{rot}")


def test_fp8_rotation_lowers_error_against_exact_attention():
    # the page's claim on synthetic outlier inputs (1 % of the Q and K entries with standard
    # deviation 10), measured end to end on the GPU: the rotated path's O is closer to the
    # exact float64 attention of the 16-bit inputs than the unrotated path's
    B, H, n, d = 2, 4, 512, 128
    q = with_outliers((B, H, n, d), torch.bfloat16, 701, 0.01, 10.0)
    k = with_outliers((B, H, n, d), torch.bfloat16, 702, 0.01, 10.0)
    v = normal((B, H, n, d), torch.bfloat16, 703)
    scale = 1.0 / math.sqrt(d)
    exact, _ = oracle.attention_forward(np64(q), np64(k), np64(v), scale, causal=True)
    errs = []
    for s in (None, random_signs(d, 704)):
        o, _ = fa.fa_attention_fp8(q.to(DEV), k.to(DEV), v.to(DEV), causal=True, scale=scale,
                                   signs=s)
        torch.cuda.synchronize()
        errs.append(float(np.sqrt(np.mean((np64(o) - exact) ** 2))))
    assert errs[1] < errs[0], errs


def test_fp8_full_size_sampled_rows():
    # the bf16 causal B2 H16 N8192 d128 workload, rotated; two whole heads' operands
    # quantised by the oracle, sampled rows compared
    w = WORKLOADS[5]
    q, k, v, _ = qkv_inputs(w, with_dout=False)
    s = random_signs(w.d, 705)
    o, lse = fa.fa_attention_fp8(q.to(DEV), k.to(DEV), v.to(DEV), causal=True, scale=w.scale,
                                 signs=s)
    torch.cuda.synchronize()
    assert torch.isfinite(o).all()
    rows = sample_rows(w.N_q, 24, 706)
    for (b, h) in ((0, 0), (1, 11)):
        one = lambda t: t[b:b + 1, h:h + 1]  # noqa: E731
        qh, kh, vh, div = F.fp8_attention_operands(np64(one(q)), np64(one(k)), np64(one(v)), s)
        o_ref, lse_ref = oracle.attention_forward_rows(qh, kh, vh, w.scale / div, rows, 0, 0,
                                                       causal=True)
        full_o = np.zeros((1, 1, w.N_q, w.d))
        full_l = np.zeros((1, 1, w.N_q))
        full_o[0, 0, rows] = o_ref
        full_l[0, 0, rows] = lse_ref
        check_fp8(one(o), one(lse), qh, kh, vh, div, full_o, full_l, w.scale, True,
                  f"fp8 N8192 b{b} h{h}", rows=rows)
