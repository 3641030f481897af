"""GPU parity of the block-sparse forward (a block bitmap in the mask descriptor).

Blocks of block_q query rows by block_k keys whose bitmap byte is zero are masked; the
library never loads or computes the tiles inside them. Results must meet fa_fwd's
tolerances against the float64 oracle, for bitmaps shared by all heads, per head and per
(batch, head), with ragged lengths, causal masking, key ranges and bias.
"""

import math

import numpy as np
import pytest
import torch

import oracle
from synth import key_ranges, normal
from tests.util import assert_fwd_close, np64, sample_rows

pytestmark = pytest.mark.gpu

fa = pytest.importorskip("exact_io_aware_flash_amd")
DEV = "cuda:0"


def bitmap(shape, density, seed):
    return (np.random.default_rng(seed).random(shape) < density).astype(np.uint8)


def run(q, k, v, bm, bq, bk, split=None, **kw):
    m = (torch.from_numpy(bm).to(DEV), bq, bk)
    if split is None:
        o, lse = fa.fa_fwd(q.to(DEV), k.to(DEV), v.to(DEV), block_mask=m, **kw)
    else:
        o, lse = fa.fa_fwd_split(q.to(DEV), k.to(DEV), v.to(DEV), block_mask=m, n_split=split, **kw)
    torch.cuda.synchronize()
    return o, lse


CASES = [
    # dtype, d, causal, nq, nk, bq, bk, density, layout
    (torch.bfloat16, 128, False, 300, 520, 64, 64, 0.5, "shared"),
    (torch.bfloat16, 128, True, 520, 520, 128, 64, 0.6, "head"),
    (torch.float16, 64, False, 257, 700, 64, 192, 0.5, "batch_head"),
    (torch.float16, 128, True, 1000, 1000, 192, 128, 0.4, "shared"),
    (torch.bfloat16, 64, True, 640, 320, 64, 64, 0.7, "head"),
    (torch.bfloat16, 128, False, 64, 2000, 64, 128, 0.3, "shared"),
]


@pytest.mark.parametrize("dtype,d,causal,nq,nk,bq,bk,density,layout", CASES)
def test_block_sparse_matches_oracle(dtype, d, causal, nq, nk, bq, bk, density, layout):
    B, H = 2, 3
    seed = 9001 + nq + 7 * nk + bq + bk + d
    q, k, v = (normal((B, H, n, d), dtype, seed + i) for i, n in enumerate((nq, nk, nk)))
    nbq, nbk = -(-nq // bq), -(-nk // bk)
    shape = {"shared": (nbq, nbk), "head": (H, nbq, nbk), "batch_head": (B, H, nbq, nbk)}[layout]
    bm = bitmap(shape, density, seed + 5)
    scale = 1.0 / math.sqrt(d)
    o, lse = run(q, k, v, bm, bq, bk, scale=scale, causal=causal)
    o_ref, lse_ref = oracle.attention_forward(np64(q), np64(k), np64(v), scale, causal=causal,
                                              block_mask=(bm, bq, bk))
    assert_fwd_close(np64(o), np64(lse), o_ref, lse_ref, dtype,
                     f"block-sparse {layout} {nq}x{nk} {bq}x{bk} c{causal}")


@pytest.mark.parametrize("causal", [False, True])
def test_block_sparse_with_ranges_and_bias(causal):
    B, H, nq, nk, d = 1, 4, 384, 640, 128
    dtype = torch.bfloat16
    q, k, v = (normal((B, H, n, d), dtype, 9100 + i) for i, n in enumerate((nq, nk, nk)))
    ks, ke = key_ranges(nq, nk, seed=9104, block=64, width=320, jitter=32)
    bm = bitmap((H, 3, 10), 0.6, 9105)
    bm[1, 1, :] = 0  # an empty block row in head 1: its rows see nothing
    slopes = [-0.02, 0.01, -0.05, 0.0]
    scale = 1.0 / math.sqrt(d)
    o, lse = run(q, k, v, bm, 128, 64, scale=scale, causal=causal, bias_slopes=slopes,
                 key_start=ks.to(DEV), key_end=ke.to(DEV))
    o_ref, lse_ref = oracle.attention_forward(
        np64(q), np64(k), np64(v), scale, causal=causal,
        bias_slopes=np.float32(slopes).astype(np.float64), key_start=ks.numpy(),
        key_end=ke.numpy(), block_mask=(bm, 128, 64))
    assert np.all(np.isneginf(lse_ref[0, 1, 128:256]))
    assert_fwd_close(np64(o), np64(lse), o_ref, lse_ref, dtype, f"block-sparse ranges bias c{causal}")


def test_all_zero_bitmap_gives_empty_rows():
    B, H, nq, nk, d = 1, 2, 200, 300, 64
    q, k, v = (normal((B, H, n, d), torch.float16, 9200 + i) for i, n in enumerate((nq, nk, nk)))
    o, lse = run(q, k, v, np.zeros((4, 5), dtype=np.uint8), 64, 64)
    assert torch.all(o == 0) and torch.all(torch.isneginf(lse))


def test_all_one_bitmap_equals_dense():
    B, H, nq, nk, d = 2, 2, 333, 777, 128
    q, k, v = (normal((B, H, n, d), torch.bfloat16, 9300 + i) for i, n in enumerate((nq, nk, nk)))
    o1, l1 = run(q, k, v, np.ones((6, 13), dtype=np.uint8), 64, 64, causal=True)
    o0, l0 = fa.fa_fwd(q.to(DEV), k.to(DEV), v.to(DEV), causal=True)
    torch.cuda.synchronize()
    assert torch.equal(o1, o0) and torch.equal(l1, l0)


@pytest.mark.parametrize("nq,nk,split", [(16, 4096, 0), (1, 3000, 5), (300, 2000, 3)])
def test_block_sparse_split_forward(nq, nk, split):
    B, H, d = 2, 3, 128
    dtype = torch.bfloat16
    q, k, v = (normal((B, H, n, d), dtype, 9400 + nq + i) for i, n in enumerate((nq, nk, nk)))
    bq, bk = 64, 128
    bm = bitmap((B, H, -(-nq // bq), -(-nk // bk)), 0.5, 9405 + nk)
    scale = 1.0 / math.sqrt(d)
    o, lse = run(q, k, v, bm, bq, bk, split=split, scale=scale, causal=True)
    o_ref, lse_ref = oracle.attention_forward(np64(q), np64(k), np64(v), scale, causal=True,
                                              block_mask=(bm, bq, bk))
    assert_fwd_close(np64(o), np64(lse), o_ref, lse_ref, dtype, f"block-sparse split {nq}x{nk}")


def test_block_sparse_many_heads():
    # a grid large enough for the 8-wave workgroup form
    B, H, nq, nk, d = 16, 64, 520, 520, 128
    dtype = torch.bfloat16
    q, k, v = (normal((B, H, n, d), dtype, 9500 + i) for i, n in enumerate((nq, nk, nk)))
    bm = bitmap((H, 5, 5), 0.5, 9505)
    scale = 1.0 / math.sqrt(d)
    o, lse = run(q, k, v, bm, 128, 128, scale=scale, causal=True)
    for (b, h) in ((0, 0), (9, 31), (15, 63)):
        one = lambda t: np64(t[b:b + 1, h:h + 1])  # noqa: E731
        o_ref, lse_ref = oracle.attention_forward(one(q), one(k), one(v), scale, causal=True,
                                                  block_mask=(bm[h], 128, 128))
        assert_fwd_close(one(o), np64(lse[b:b + 1, h:h + 1]), o_ref, lse_ref, dtype,
                         f"block-sparse many heads b{b} h{h}")


def test_block_sparse_full_size_n8192():
    # C5-sized heads with half of the 128 x 128 blocks kept; sampled rows of two heads
    B, H, n, d = 2, 16, 8192, 128
    dtype = torch.bfloat16
    q, k, v = (normal((B, H, n, d), dtype, 9600 + i) for i in range(3))
    bm = bitmap((H, 64, 64), 0.5, 9603)
    scale = 1.0 / math.sqrt(d)
    o, lse = run(q, k, v, bm, 128, 128, scale=scale, causal=True)
    for (b, h) in ((0, 0), (1, 11)):
        rows = sample_rows(n, 48, seed=b * 100 + h)
        one = lambda t: np64(t[b:b + 1, h:h + 1])  # noqa: E731
        o_ref, lse_ref = oracle.attention_forward_rows(one(q), one(k), one(v), scale, rows, 0, 0,
                                                       True, None, None, None, (bm[h], 128, 128))
        o_g = np64(o[b, h][torch.as_tensor(rows)])
        l_g = np64(lse[b, h][torch.as_tensor(rows)])
        assert_fwd_close(o_g, l_g, o_ref, lse_ref, dtype, f"block-sparse N8192 b{b} h{h}")
