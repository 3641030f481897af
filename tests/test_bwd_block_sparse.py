"""GPU parity of the block-sparse backward (a block bitmap in the mask descriptor).

The gradients of attention under a block bitmap are those of the masked scores: blocks
whose byte is zero contribute nothing to dQ, dK or dV, and the library never loads the
tiles inside them. Results must meet fa_bwd's tolerances against the float64 oracle
gradients, for bitmaps shared by all heads, per head and per (batch, head), with ragged
lengths, causal masking, key ranges and bias.
"""

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


def bitmap(shape, density, seed):
    return (np.random.default_rng(seed).random(shape) < density).astype(np.uint8)


def fwd_bwd(q, k, v, do, bm=None, **kw):
    q, k, v, do = (t.to(DEV) for t in (q, k, v, do))
    if bm is not None:
        kw["block_mask"] = (torch.from_numpy(bm[0]).to(DEV), bm[1], bm[2])
    o, lse = fa.fa_fwd(q, k, v, **kw)
    dq, dk, dv = fa.fa_bwd(do, q, k, v, o, lse, **kw)
    torch.cuda.synchronize()
    return dq, dk, dv


def check_grads(got, want, what, tol=GRAD_TOL):
    for name, g, w in zip(("dQ", "dK", "dV"), got, want):
        g = np64(g)
        assert np.isfinite(g).all(), f"{what}: non-finite {name}"
        worst = float(np.abs(g - w).max()) if g.size else 0.0
        assert worst <= tol, f"{what}: {name} max err {worst:.3e} > {tol}"


CASES = [
    # dtype, d, causal, nq, nk, bq, bk, density, layout
    (torch.bfloat16, 128, False, 300, 520, 64, 64, 0.5, "shared"),
    (torch.bfloat16, 128, True, 520, 520, 128, 64, 0.6, "head"),
    (torch.float16, 64, False, 257, 700, 64, 192, 0.5, "batch_head"),
    (torch.float16, 128, True, 1000, 1000, 192, 128, 0.4, "shared"),
    (torch.bfloat16, 64, True, 640, 320, 64, 64, 0.7, "head"),
    (torch.bfloat16, 128, False, 64, 2000, 64, 128, 0.3, "shared"),
    (torch.float16, 64, True, 333, 1100, 128, 256, 0.5, "batch_head"),
]


@pytest.mark.parametrize("dtype,d,causal,nq,nk,bq,bk,density,layout", CASES)
def test_block_sparse_gradients_match_oracle(dtype, d, causal, nq, nk, bq, bk, density, layout):
    B, H = 2, 3
    seed = 19001 + nq + 7 * nk + bq + bk + d
    q, k, v, do = (normal((B, H, n, d), dtype, seed + i) for i, n in enumerate((nq, nk, nk, nq)))
    nbq, nbk = -(-nq // bq), -(-nk // bk)
    shape = {"shared": (nbq, nbk), "head": (H, nbq, nbk), "batch_head": (B, H, nbq, nbk)}[layout]
    bm = bitmap(shape, density, seed + 5)
    scale = 1.0 / math.sqrt(d)
    got = fwd_bwd(q, k, v, do, (bm, bq, bk), scale=scale, causal=causal)
    want = oracle.attention_backward(np64(q), np64(k), np64(v), np64(do), scale, causal=causal,
                                     block_mask=(bm, bq, bk))
    check_grads(got, want, f"block-sparse bwd {layout} {nq}x{nk} {bq}x{bk} c{causal} d{d}")


@pytest.mark.parametrize("causal", [False, True])
def test_block_sparse_gradients_with_ranges_and_bias(causal):
    B, H, nq, nk, d = 1, 4, 384, 640, 128
    dtype = torch.bfloat16
    q, k, v, do = (normal((B, H, n, d), dtype, 19100 + i) for i, n in enumerate((nq, nk, nk, nq)))
    ks, ke = key_ranges(nq, nk, seed=19104, block=64, width=320, jitter=32)
    bm = bitmap((H, 3, 10), 0.6, 19105)
    bm[1, 1, :] = 0  # an empty block row in head 1: its rows get no gradient
    bm[2, :, 4] = 0  # an empty block column in head 2: its keys get no gradient
    slopes = [-0.02, 0.01, -0.05, 0.0]
    scale = 1.0 / math.sqrt(d)
    got = fwd_bwd(q, k, v, do, (bm, 128, 64), scale=scale, causal=causal, bias_slopes=slopes,
                  key_start=ks.to(DEV), key_end=ke.to(DEV))
    want = oracle.attention_backward(
        np64(q), np64(k), np64(v), np64(do), scale, causal=causal,
        bias_slopes=np.float32(slopes).astype(np.float64), key_start=ks.numpy(),
        key_end=ke.numpy(), block_mask=(bm, 128, 64))
    assert not want[0][0, 1, 128:256].any() and not want[1][0, 2, 256:320].any()
    check_grads(got, want, f"block-sparse bwd ranges bias c{causal}")


def test_all_zero_bitmap_gives_zero_gradients():
    B, H, nq, nk, d = 1, 2, 200, 300, 64
    q, k, v, do = (normal((B, H, n, d), torch.float16, 19200 + i)
                   for i, n in enumerate((nq, nk, nk, nq)))
    got = fwd_bwd(q, k, v, do, (np.zeros((4, 5), dtype=np.uint8), 64, 64))
    for g in got:
        assert torch.all(g == 0)


def test_all_one_bitmap_equals_dense():
    # d = 128 uses the same tiles with and without the bitmap, so the sums agree bit for bit
    B, H, nq, nk, d = 2, 2, 333, 777, 128
    q, k, v, do = (normal((B, H, n, d), torch.bfloat16, 19300 + i)
                   for i, n in enumerate((nq, nk, nk, nq)))
    g1 = fwd_bwd(q, k, v, do, (np.ones((6, 13), dtype=np.uint8), 64, 64), causal=True)
    g0 = fwd_bwd(q, k, v, do, causal=True)
    for a, b in zip(g1, g0):
        assert torch.equal(a, b)


def test_block_sparse_backward_is_deterministic():
    B, H, n, d = 1, 4, 700, 128
    q, k, v, do = (normal((B, H, n, d), torch.bfloat16, 19400 + i) for i in range(4))
    bm = bitmap((H, 11, 11), 0.5, 19405)
    a = fwd_bwd(q, k, v, do, (bm, 64, 64), causal=True)
    b = fwd_bwd(q, k, v, do, (bm, 64, 64), causal=True)
    for x, y in zip(a, b):
        assert torch.equal(x, y)


def test_block_sparse_many_heads():
    # a grid wide enough for the XCD-aware workgroup order
    B, H, nq, nk, d = 8, 16, 520, 520, 128
    dtype = torch.bfloat16
    q, k, v, do = (normal((B, H, n, d), dtype, 19500 + i) for i, n in enumerate((nq, nk, nk, nq)))
    bm = bitmap((B, H, 9, 5), 0.5, 19505)
    scale = 1.0 / math.sqrt(d)
    got = fwd_bwd(q, k, v, do, (bm, 64, 128), scale=scale, causal=True)
    for (b, h) in ((0, 0), (3, 7), (7, 15)):
        one = lambda t: np64(t[b:b + 1, h:h + 1])  # noqa: E731
        want = oracle.attention_backward(one(q), one(k), one(v), one(do), scale, causal=True,
                                         block_mask=(bm[b:b + 1, h:h + 1], 64, 128))
        check_grads(tuple(g[b:b + 1, h:h + 1] for g in got), want, f"many heads b{b} h{h}")


def test_block_sparse_full_size_backward():
    # the bf16 causal N = 8192 d = 128 workload with half of its 128 x 128 blocks masked;
    # the oracle checks one whole (b, h) head
    w = WORKLOADS[5]
    q, k, v, do = qkv_inputs(w)
    nb = -(-w.N_q // 128)
    bm = bitmap((w.H, nb, nb), 0.5, 19605)
    got = fwd_bwd(q, k, v, do, (bm, 128, 128), scale=w.scale, causal=True)
    for g in got:
        assert torch.isfinite(g).all()
    b, h = 1, 5
    one = lambda t: np64(t[b:b + 1, h:h + 1])  # noqa: E731
    want = oracle.attention_backward(one(q), one(k), one(v), one(do), w.scale, causal=True,
                                     block_mask=(bm[h:h + 1], 128, 128), max_chunk_elems=1 << 25)
    check_grads(tuple(g[b:b + 1, h:h + 1] for g in got), want, f"{w.name} block-sparse b{b} h{h}")
