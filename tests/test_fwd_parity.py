"""GPU forward parity against the fp64 CPU oracle (through the C ABI)."""

import math

import numpy as np
import pytest
import torch

import oracle
from synth import WORKLOADS, key_ranges, normal, qkv_inputs, seed_for
from tests.util import assert_fwd_close, np64, sample_rows

pytestmark = pytest.mark.gpu

fa = pytest.importorskip("exact_io_aware_flash_amd")
DEV = "cuda:0"


def run(q, k, v, **kw):
    o, lse = fa.fa_fwd(q.to(DEV), k.to(DEV), v.to(DEV), **kw)
    torch.cuda.synchronize()
    return o, lse


def ranges_dev(ks, ke):
    return ks.to(DEV), ke.to(DEV)


# ---------------------------------------------------------------------------
# the single-head fp32 workload, full oracle
# ---------------------------------------------------------------------------
def test_fp32_single_head_full():
    w = WORKLOADS[1]
    q, k, v, _ = qkv_inputs(w)
    o, lse = run(q, k, v, scale=w.scale)
    o_ref, lse_ref = oracle.attention_forward(np64(q), np64(k), np64(v), w.scale)
    assert_fwd_close(np64(o), np64(lse), o_ref, lse_ref, torch.float32, "fp32 B1H1N256d64")


# ---------------------------------------------------------------------------
# small shapes spanning several tiles, ragged tails, N_q != N_k
# ---------------------------------------------------------------------------
SHAPES = [(1, 1), (2, 3), (63, 65), (64, 64), (129, 127), (300, 300), (257, 520), (520, 257)]


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float16, torch.float32])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("nq,nk", SHAPES)
def test_small_shapes(dtype, d, causal, nq, nk):
    B, H = 1, 2
    seed = nq * 7919 + nk * 31 + d + (1 if causal else 0)
    q = normal((B, H, nq, d), dtype, seed)
    k = normal((B, H, nk, d), dtype, seed + 1)
    v = normal((B, H, nk, d), dtype, seed + 2)
    scale = 1.0 / math.sqrt(d)
    o, lse = run(q, k, v, scale=scale, causal=causal)
    o_ref, lse_ref = oracle.attention_forward(np64(q), np64(k), np64(v), scale, causal=causal)
    assert_fwd_close(np64(o), np64(lse), o_ref, lse_ref, dtype, f"{dtype} d{d} c{causal} {nq}x{nk}")


@pytest.mark.parametrize("dtype,d", [(torch.bfloat16, 128), (torch.float16, 64),
                                     (torch.float32, 64)])
@pytest.mark.parametrize("causal", [False, True])
def test_bias_and_key_ranges_small(dtype, d, causal):
    B, H, nq, nk = 2, 3, 700, 650
    q = normal((B, H, nq, d), dtype, 11)
    k = normal((B, H, nk, d), dtype, 12)
    v = normal((B, H, nk, d), dtype, 13)
    ks, ke = key_ranges(nq, nk, seed=14, block=128, width=nk // 2, jitter=64)
    ks, ke = ks.clone(), ke.clone()
    # out-of-range and empty intervals are legal inputs
    ks[3], ke[3] = -50, 10
    ks[4], ke[4] = 600, 900
    ks[5], ke[5] = 300, 300
    ks[6], ke[6] = 500, 100
    ks[699], ke[699] = 0, nk
    slopes = [-0.1 / 64, -0.05, 0.01]
    scale = 1.0 / math.sqrt(d)
    kd, ked = ranges_dev(ks, ke)
    o, lse = run(q, k, v, scale=scale, causal=causal, bias_slopes=slopes, key_start=kd, key_end=ked)
    o_ref, lse_ref = oracle.attention_forward(np64(q), np64(k), np64(v), scale, causal=causal,
                                              bias_slopes=np.float32(slopes).astype(np.float64),
                                              key_start=ks.numpy(), key_end=ke.numpy())
    assert_fwd_close(np64(o), np64(lse), o_ref, lse_ref, dtype, f"bias+range {dtype} d{d}")


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
def test_bias_only_and_range_only(dtype):
    B, H, n, d = 1, 2, 333, 64
    q, k, v = (normal((B, H, n, d), dtype, s) for s in (21, 22, 23))
    scale = 0.11
    o, lse = run(q, k, v, scale=scale, bias_slopes=0.02)
    o_ref, lse_ref = oracle.attention_forward(np64(q), np64(k), np64(v), scale,
                                              bias_slopes=float(np.float32(0.02)))
    assert_fwd_close(np64(o), np64(lse), o_ref, lse_ref, dtype, "bias only")
    ks, ke = key_ranges(n, n, seed=24, block=64, width=100, jitter=30)
    o, lse = run(q, k, v, scale=scale, key_start=ks.to(DEV), key_end=ke.to(DEV))
    o_ref, lse_ref = oracle.attention_forward(np64(q), np64(k), np64(v), scale,
                                              key_start=ks.numpy(), key_end=ke.numpy())
    assert_fwd_close(np64(o), np64(lse), o_ref, lse_ref, dtype, "range only")


def test_all_rows_masked():
    B, H, n, d = 1, 1, 200, 128
    q, k, v = (normal((B, H, n, d), torch.bfloat16, s) for s in (31, 32, 33))
    ks = torch.full((n,), 5, dtype=torch.int32)
    ke = torch.full((n,), 5, dtype=torch.int32)
    o, lse = run(q, k, v, key_start=ks.to(DEV), key_end=ke.to(DEV))
    assert torch.all(o == 0) and torch.all(torch.isneginf(lse))


def test_causal_more_queries_than_keys_gives_empty_rows():
    B, H, nq, nk, d = 1, 2, 300, 100, 64
    q = normal((B, H, nq, d), torch.float16, 41)
    k = normal((B, H, nk, d), torch.float16, 42)
    v = normal((B, H, nk, d), torch.float16, 43)
    o, lse = run(q, k, v, causal=True)
    o_ref, lse_ref = oracle.attention_forward(np64(q), np64(k), np64(v), 1 / 8, causal=True)
    assert np.isneginf(lse_ref[0, 0, :199]).all()
    assert_fwd_close(np64(o), np64(lse), o_ref, lse_ref, torch.float16, "causal Nq>Nk")


def test_large_magnitude_scores_stay_finite():
    # scores up to ~1e3: the running max must keep every exponential in range
    B, H, n, d = 1, 1, 400, 64
    q = normal((B, H, n, d), torch.bfloat16, 51, factor=6.0)
    k = normal((B, H, n, d), torch.bfloat16, 52, factor=6.0)
    v = normal((B, H, n, d), torch.bfloat16, 53)
    o, lse = run(q, k, v, scale=1.0, causal=True)
    o_ref, lse_ref = oracle.attention_forward(np64(q), np64(k), np64(v), 1.0, causal=True)
    assert_fwd_close(np64(o), np64(lse), o_ref, lse_ref, torch.bfloat16, "large scores")


@pytest.mark.parametrize("dtype,d", [(torch.bfloat16, 128), (torch.float16, 64)])
@pytest.mark.parametrize("causal", [False, True])
def test_scores_growing_along_keys(dtype, d, causal):
    # Key j carries 8*j in coordinate 0 and every query a positive coordinate 0 (up to 4),
    # so each 64-key tile raises a row's scores by up to ~260 (log2 units) over the last:
    # the running max must move on almost every tile, by more than 128 on the rows whose
    # first probabilities against the stale max overflow to infinity.
    B, H, n = 1, 2, 700
    q = normal((B, H, n, d), torch.float32, 61)
    k = normal((B, H, n, d), torch.float32, 62)
    q[..., 0] = torch.linspace(0.0, 4.0, n)
    k[..., 0] = 8.0 * torch.arange(n, dtype=torch.float32)
    q, k = q.to(dtype), k.to(dtype)
    v = normal((B, H, n, d), dtype, 63)
    o, lse = run(q, k, v, causal=causal)
    o_ref, lse_ref = oracle.attention_forward(np64(q), np64(k), np64(v), 1 / math.sqrt(d),
                                              causal=causal)
    assert_fwd_close(np64(o), np64(lse), o_ref, lse_ref, dtype, f"growing scores c{causal}")


def test_forward_is_deterministic():
    w = WORKLOADS[2].scaled(B=1, H=4, N_q=1000, N_k=1000)
    q, k, v, _ = qkv_inputs(w)
    o1, l1 = run(q, k, v, causal=True)
    o2, l2 = run(q, k, v, causal=True)
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


# ---------------------------------------------------------------------------
# key-range summary (integer, bit-exact)
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("block", [1, 64, 128, 1000])
def test_mask_summary_bit_exact(block):
    n_q, n_k = 5000, 4096
    ks, ke = key_ranges(n_q, n_k, seed=61, block=128, width=2048, jitter=64)
    ks, ke = ks.clone(), ke.clone()
    ks[7], ke[7] = -9, 99999
    out = fa.fa_mask_summary(ks.to(DEV), ke.to(DEV), n_k, block)
    torch.cuda.synchronize()
    want = oracle.row_block_summary(ks.numpy(), ke.numpy(), n_k, block)
    assert np.array_equal(out.cpu().numpy().astype(np.int64), want)


# ---------------------------------------------------------------------------
# many heads of ragged length: for d = 128 the library picks the larger workgroup only
# for grids with several 256-row blocks per compute unit, so small shapes alone would not
# reach it; whole sampled heads are checked
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("causal,bias,nq,nk", [(True, False, 300, 300), (False, False, 257, 520),
                                               (True, True, 520, 257), (False, True, 300, 300)])
def test_many_heads_ragged(causal, bias, nq, nk):
    B, H, d = 16, 64, 128
    dtype = torch.bfloat16
    seed = 4099 + nq + 3 * nk + (7 if causal else 0) + (11 if bias else 0)
    q = normal((B, H, nq, d), dtype, seed)
    k = normal((B, H, nk, d), dtype, seed + 1)
    v = normal((B, H, nk, d), dtype, seed + 2)
    scale = 1.0 / math.sqrt(d)
    slopes = [-0.02 - 0.001 * i for i in range(H)] if bias else None
    kw = dict(scale=scale, causal=causal)
    if bias:
        kw.update(bias_slopes=slopes)
    o, lse = run(q, k, v, **kw)
    for (b, h) in ((0, 0), (7, 33), (15, 63)):
        one = lambda t: np64(t[b:b + 1, h:h + 1])  # noqa: E731
        o_ref, lse_ref = oracle.attention_forward(
            one(q), one(k), one(v), scale, causal=causal,
            bias_slopes=None if slopes is None else np.float32([slopes[h]]).astype(np.float64))
        assert_fwd_close(one(o), np64(lse[b:b + 1, h:h + 1]), o_ref, lse_ref, dtype,
                         f"many heads b{b} h{h} {nq}x{nk} c{causal} bias{bias}")


# ---------------------------------------------------------------------------
# full-size workloads: sampled rows of sampled heads against the oracle
# ---------------------------------------------------------------------------
def _full_config_check(wid, heads, nrows):
    w = WORKLOADS[wid]
    q, k, v, _ = qkv_inputs(w, with_dout=False)
    kw = dict(scale=w.scale, causal=w.causal)
    ks = ke = None
    slopes = None
    if w.key_range:
        ks, ke = key_ranges(w.N_q, w.N_k, seed_for(wid, 9), block=128, width=w.N_k // 2, jitter=64)
        kw.update(key_start=ks.to(DEV), key_end=ke.to(DEV))
    if w.bias_slope is not None:
        slopes = float(np.float32(w.bias_slope))
        kw.update(bias_slopes=w.bias_slope)
    o, lse = run(q, k, v, **kw)
    assert torch.isfinite(o).all()
    for (b, h) in heads:
        rows = sample_rows(w.N_q, nrows, seed=b * 100 + h)
        one = lambda t: np64(t[b:b + 1, h:h + 1])  # noqa: E731  (one head, exact up-cast)
        o_ref, lse_ref = oracle.attention_forward_rows(
            one(q), one(k), one(v), w.scale, rows, 0, 0, w.causal, slopes,
            None if ks is None else ks.numpy(), None if ke is None else ke.numpy())
        o_g = np64(o[b, h][torch.as_tensor(rows)])
        l_g = np64(lse[b, h][torch.as_tensor(rows)])
        assert_fwd_close(o_g, l_g, o_ref, lse_ref, w.torch_dtype, f"{w.name} b{b} h{h}")


def test_full_causal_bf16_n2048():
    _full_config_check(2, [(0, 0), (3, 15), (1, 7)], 96)


def test_full_long_sequence_fp16_n23400():
    _full_config_check(3, [(0, 0), (0, 11)], 48)


def test_full_bias_key_range_bf16_n8192():
    _full_config_check(4, [(0, 0), (1, 7)], 64)


def test_full_causal_bf16_n8192_forward():
    _full_config_check(5, [(0, 0), (1, 15)], 64)


def test_long_sequence_memory_stays_linear():
    # the fp16 score matrix of this workload would be ~13 GB; the kernel must only
    # need its inputs and outputs
    w = WORKLOADS[3]
    q, k, v, _ = qkv_inputs(w, with_dout=False)
    q, k, v = q.to(DEV), k.to(DEV), v.to(DEV)
    o = torch.empty_like(q)
    lse = torch.empty(q.shape[:3], dtype=torch.float32, device=DEV)
    torch.cuda.synchronize()
    torch.cuda.reset_peak_memory_stats()
    base = torch.cuda.memory_allocated()
    fa.fa_fwd(q, k, v, out=o, lse=lse)
    torch.cuda.synchronize()
    assert torch.cuda.max_memory_allocated() - base == 0
    score_bytes = w.H * w.N_q * w.N_k * 2
    io_bytes = 4 * q.numel() * 2 + lse.numel() * 4
    assert io_bytes * 50 < score_bytes
