"""Race check: the library built with FA_SYNC_CHECK=1 (every ring step waits for all of its
loads and passes a full workgroup barrier right after issuing the next tile, so copies do
not overlap compute and no wave runs ahead) must give the same bits as the normal build.

A difference would mean a result that depends on timing: an LDS stage reused before every
wave finished with it, a load consumed before it landed, a missing barrier. Both
libraries are built from the same sources by build() (libfa.so, libfa_synccheck.so); the
inputs cover every ring: 16-bit forward (plain, split, bias tensor, block bitmap), the
16-bit backward passes (with dbias, dslopes and the atomic dQ form, whose dQ is compared
against the bound of the oracle test instead, the order of its atomic additions being
free), float32 forward and backward, and the FP8 forward.
"""

import contextlib
import math
import os

import numpy as np
import pytest
import torch

from synth import bias_tensor, key_ranges, normal, random_signs

pytestmark = pytest.mark.gpu

fa = pytest.importorskip("exact_io_aware_flash_amd")
from exact_io_aware_flash_amd.build import SYNC_CHECK_LIB  # noqa: E402

DEV = "cuda:0"


@contextlib.contextmanager
def library(path):
    old = (fa._LIB, fa._LIB_PATH)
    fa._LIB, fa._LIB_PATH = None, path
    try:
        fa.load_library()
        yield
    finally:
        fa._LIB, fa._LIB_PATH = old


def both(fn):
    """fn() with the normal library, then with the race-check library (tensors cloned)."""
    assert os.path.exists(SYNC_CHECK_LIB), "race-check library missing: run build()"
    a = [t.clone() for t in fn()]
    torch.cuda.synchronize()
    with library(SYNC_CHECK_LIB):
        b = [t.clone() for t in fn()]
        torch.cuda.synchronize()
    return a, b


def assert_same(a, b, what):
    for i, (x, y) in enumerate(zip(a, b)):
        assert torch.equal(x, y), f"{what}: output {i} differs between the builds"


def inputs(dtype, B, H, nq, nk, d, seed):
    return tuple(normal((B, H, n, d), dtype, seed + i).to(DEV)
                 for i, n in enumerate((nq, nk, nk, nq)))


@pytest.mark.parametrize("dtype,d,causal", [(torch.bfloat16, 128, True),
                                            (torch.float16, 64, False),
                                            (torch.float32, 128, True)])
def test_forward_and_backward_same_bits(dtype, d, causal):
    q, k, v, do = inputs(dtype, 2, 3, 700, 650, d, 31000 + d)

    def run():
        o, lse = fa.fa_fwd(q, k, v, causal=causal)
        return (o, lse) + tuple(fa.fa_bwd(do, q, k, v, o, lse, causal=causal))
    assert_same(*both(run), f"{dtype} d{d} c{causal}")


def test_split_ranges_slope_and_dslopes_same_bits():
    q, k, v, do = inputs(torch.bfloat16, 1, 3, 520, 1500, 128, 31100)
    ks, ke = key_ranges(520, 1500, seed=31105, block=64, width=700, jitter=32)
    kw = dict(causal=True, bias_slopes=[-0.02, 0.01, -0.05], key_start=ks.to(DEV),
              key_end=ke.to(DEV))

    def run():
        o, lse = fa.fa_fwd(q, k, v, **kw)
        o2, lse2 = fa.fa_fwd_split(q[:, :, :16].contiguous(), k, v, n_split=5,
                                   **dict(kw, key_start=None, key_end=None))
        ds = torch.zeros(3, dtype=torch.float32, device=DEV)
        g = fa.fa_bwd(do, q, k, v, o, lse, dslopes=ds, **kw)
        return (o, lse, o2, lse2, ds) + tuple(g)
    assert_same(*both(run), "split / ranges / slope")


def test_bias_tensor_dbias_and_bitmap_same_bits():
    B, H, nq, nk, d = 2, 2, 400, 460, 128
    q, k, v, do = inputs(torch.bfloat16, B, H, nq, nk, d, 31200)
    bias = bias_tensor((1, H, nq, nk), 31205, 2.0, 0.05).to(DEV)
    bm = torch.from_numpy((np.random.default_rng(31206).random((H, 7, 8)) < 0.6)
                          .astype(np.uint8)).to(DEV)

    def run():
        o, lse = fa.fa_fwd(q, k, v, causal=True, bias=bias)
        db = torch.empty((B, H, nq, nk), dtype=torch.float32, device=DEV)
        g = fa.fa_bwd(do, q, k, v, o, lse, causal=True, bias=bias, dbias=db)
        dbs = torch.empty((1, H, nq, nk), dtype=torch.float32, device=DEV)
        fa.fa_bwd(do, q, k, v, o, lse, causal=True, bias=bias, dbias=dbs)
        o3, lse3 = fa.fa_fwd(q, k, v, causal=False, block_mask=(bm, 64, 64))
        g3 = fa.fa_bwd(do, q, k, v, o3, lse3, causal=False, block_mask=(bm, 64, 64))
        return (o, lse, db, dbs, o3, lse3) + tuple(g) + tuple(g3)
    assert_same(*both(run), "bias tensor / dbias / bitmap")


def test_atomic_dq_form_dk_dv_same_bits():
    q, k, v, do = inputs(torch.bfloat16, 1, 2, 900, 900, 128, 31300)
    ph = fa.FA_BWD_PREP | fa.FA_BWD_DKDV | fa.FA_BWD_DQ_ATOMIC

    def run():
        o, lse = fa.fa_fwd(q, k, v, causal=True)
        dq, dk, dv = fa.fa_bwd(do, q, k, v, o, lse, causal=True, phases=ph)
        return dk, dv, dq
    a, b = both(run)
    assert_same(a[:2], b[:2], "atomic form dK, dV")
    assert float((a[2] - b[2]).abs().max()) <= 1e-3  # dQ: float32 additions in any order


def test_fp8_forward_same_bits():
    q, k, v, _ = inputs(torch.bfloat16, 1, 2, 700, 700, 128, 31400)
    s = random_signs(128, 31405)

    def run():
        o, lse = fa.fa_attention_fp8(q, k, v, causal=True, scale=1 / math.sqrt(128), signs=s)
        return o, lse
    assert_same(*both(run), "fp8 forward")
