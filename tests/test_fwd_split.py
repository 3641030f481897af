"""GPU parity of the split-key forward (fa_fwd_split) against the float64 oracle.

Decode-like shapes (few query rows, long key sequences): the keys of every head are cut
into ranges, each range yields a normalised partial output and LSE, and a merge launch
combines them. The result must meet the same tolerances as fa_fwd against the oracle.
"""

import math

import numpy as np
import pytest
import torch

import oracle
from synth import key_ranges, normal
from tests.util import assert_fwd_close, np64

pytestmark = pytest.mark.gpu

fa = pytest.importorskip("exact_io_aware_flash_amd")
DEV = "cuda:0"


def run_split(q, k, v, n_split, **kw):
    q, k, v = (t.to(DEV) for t in (q, k, v))
    o, lse = fa.fa_fwd_split(q, k, v, n_split=n_split, **kw)
    torch.cuda.synchronize()
    return o, lse


CASES = [
    # B, H, N_q, N_k, d, causal, dtype, n_split
    (2, 3, 1, 4096, 128, False, torch.bfloat16, 0),
    (2, 3, 16, 4096, 128, True, torch.bfloat16, 3),
    (1, 2, 40, 1000, 64, False, torch.float16, 7),
    (1, 2, 16, 300, 64, True, torch.bfloat16, 1000),
    (3, 2, 1, 130, 128, False, torch.bfloat16, 2),   # second range holds 2 keys
    (1, 1, 300, 2000, 128, True, torch.bfloat16, 4),  # two query blocks, causal diagonal
    (1, 2, 33, 5000, 128, False, torch.float16, 5),   # 33 rows: a second, 1-row wave
    # float32 inputs (float32 MFMA; 32-key tiles inside the 64-key-multiple ranges)
    (2, 3, 1, 4096, 128, True, torch.float32, 0),
    (1, 2, 40, 1000, 64, False, torch.float32, 7),
    (1, 1, 300, 2000, 128, True, torch.float32, 4),
]


@pytest.mark.parametrize("B,H,nq,nk,d,causal,dtype,n_split", CASES)
def test_split_matches_oracle(B, H, nq, nk, d, causal, dtype, n_split):
    seed = 7919 * nq + 13 * nk + d
    q = normal((B, H, nq, d), dtype, seed)
    k = normal((B, H, nk, d), dtype, seed + 1)
    v = normal((B, H, nk, d), dtype, seed + 2)
    scale = 1.0 / math.sqrt(d)
    n_eff = fa.fa_fwd_split_count(B, H, nq, nk, d, n_split)
    assert n_eff >= 1
    o, lse = run_split(q, k, v, n_split, causal=causal, scale=scale)
    o_ref, lse_ref = oracle.attention_forward(np64(q), np64(k), np64(v), scale, causal=causal)
    assert_fwd_close(np64(o), np64(lse), o_ref, lse_ref, dtype,
                     f"split n={n_split}->{n_eff} B{B}H{H} {nq}x{nk} d{d} c{causal}")


def test_split_agrees_with_unsplit_forward():
    B, H, nq, nk, d = 2, 4, 16, 8192, 128
    q, k, v = (normal((B, H, n, d), torch.bfloat16, 50 + i) for i, n in enumerate((nq, nk, nk)))
    o1, l1 = run_split(q, k, v, 8, causal=True)
    o0, l0 = fa.fa_fwd(q.to(DEV), k.to(DEV), v.to(DEV), causal=True)
    torch.cuda.synchronize()
    # both are within the oracle tolerance; against each other they differ by rounding
    assert float((o1.float() - o0.float()).abs().max()) <= 2e-2
    assert float(((l1 - l0).abs() / l0.abs().clamp(min=1.0)).max()) <= 1e-4


@pytest.mark.parametrize("causal", [False, True])
def test_split_with_bias_and_key_ranges(causal):
    # key ranges narrower than a split range leave whole ranges empty for some rows;
    # row 3 sees nothing at all (O = 0, LSE = -inf)
    B, H, nq, nk, d = 1, 3, 48, 3000, 128
    dtype = torch.bfloat16
    q, k, v = (normal((B, H, n, d), dtype, 60 + i) for i, n in enumerate((nq, nk, nk)))
    ks, ke = key_ranges(nq, nk, seed=61, block=16, width=400, jitter=64)
    ks, ke = ks.clone(), ke.clone()
    ks[3], ke[3] = 1000, 1000
    ks[5], ke[5] = -50, 70
    ks[7], ke[7] = 2900, 99999
    slopes = [-0.1 / 64, 0.02, -0.05]
    scale = 1.0 / math.sqrt(d)
    o, lse = run_split(q, k, v, 6, causal=causal, scale=scale, bias_slopes=slopes,
                       key_start=ks.to(DEV), key_end=ke.to(DEV))
    o_ref, lse_ref = oracle.attention_forward(
        np64(q), np64(k), np64(v), scale, causal=causal,
        bias_slopes=np.float32(slopes).astype(np.float64),
        key_start=ks.numpy(), key_end=ke.numpy())
    assert not np.isfinite(lse_ref[0, 0, 3])
    assert_fwd_close(np64(o), np64(lse), o_ref, lse_ref, dtype, f"split bias+range c{causal}")


def test_split_count_one_is_the_plain_forward():
    B, H, nq, nk, d = 1, 1, 8, 100, 64
    q, k, v = (normal((B, H, n, d), torch.bfloat16, 70 + i) for i, n in enumerate((nq, nk, nk)))
    assert fa.fa_fwd_split_count(B, H, nq, nk, d, 0) == 1
    o1, l1 = run_split(q, k, v, 0)
    o0, l0 = fa.fa_fwd(q.to(DEV), k.to(DEV), v.to(DEV))
    torch.cuda.synchronize()
    assert torch.equal(o1, o0) and torch.equal(l1, l0)


@pytest.mark.parametrize("B,nq,nk", [(8, 1, 8192), (1, 16, 32768)])
def test_decode_shape_full_size(B, nq, nk):
    # decode-like workloads with H=32, d=128 (causal: the queries are the last nq
    # positions), automatic split count; the oracle checks four whole heads
    H, d = 32, 128
    dtype = torch.bfloat16
    q = normal((B, H, nq, d), dtype, 80)
    k = normal((B, H, nk, d), dtype, 81)
    v = normal((B, H, nk, d), dtype, 82)
    o, lse = run_split(q, k, v, 0, causal=True)
    assert torch.isfinite(o.float()).all() and torch.isfinite(lse).all()
    scale = 1.0 / math.sqrt(d)
    for (b, h) in ((0, 0), (B // 2, 17), (B - 1, 31), (B - 1, 2)):
        one = lambda t: np64(t[b:b + 1, h:h + 1])  # noqa: E731
        o_ref, lse_ref = oracle.attention_forward(one(q), one(k), one(v), scale, causal=True)
        assert_fwd_close(one(o), np64(lse[b:b + 1, h:h + 1]), o_ref, lse_ref, dtype,
                         f"decode {nq}x{nk} b{b} h{h}")


def test_decode_few_heads_long_cache():
    # one sequence, eight heads, one query row against 131072 keys: the automatic count
    # cuts each head into many ranges, merged by one workgroup per row; the oracle checks
    # every head
    B, H, nq, nk, d = 1, 8, 1, 131072, 128
    dtype = torch.bfloat16
    assert fa.fa_fwd_split_count(B, H, nq, nk, d, 0) > 4
    q = normal((B, H, nq, d), dtype, 90)
    k = normal((B, H, nk, d), dtype, 91)
    v = normal((B, H, nk, d), dtype, 92)
    o, lse = run_split(q, k, v, 0, causal=True)
    scale = 1.0 / math.sqrt(d)
    for h in range(H):
        one = lambda t: np64(t[:, h:h + 1])  # noqa: E731
        o_ref, lse_ref = oracle.attention_forward(one(q), one(k), one(v), scale, causal=True)
        assert_fwd_close(one(o), np64(lse[:, h:h + 1]), o_ref, lse_ref, dtype,
                         f"decode B1 H8 1x{nk} h{h}")
