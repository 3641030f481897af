"""Key-range and causal boundaries at every offset inside a key tile (forward and backward).

A partial tile masks each score by comparing its key with the row's visible interval
[start, end) (and the causal limit). Here the intervals are chosen so that both ends fall
on every key offset 0..63 of a tile (so on the keys held by either half of a wave), on both
sides of the causal diagonal, including empty, one-key and whole-row intervals. Results
are compared with the float64 oracle (blog "Apakah Konteks Sehari Penuh Mengalahkan
Konteks Sepuluh Menit?", section on causal masking: a masked score contributes nothing;
FlashMask page, abstract: masks given as per-row column ranges).
"""

import math

import numpy as np
import pytest
import torch

import oracle
from synth import normal
from tests.util import GRAD_TOL, assert_fwd_close, np64

pytestmark = pytest.mark.gpu

fa = pytest.importorskip("exact_io_aware_flash_amd")
DEV = "cuda:0"


def offset_ranges(nq: int, nk: int):
    """start_i runs through every residue mod 64 (step 37 is coprime to 64), the interval
    width through 0 .. 70, with a few rows clipped at either end or covering all keys."""
    i = np.arange(nq)
    ks = (i * 37) % nk
    ke = np.minimum(ks + (i * 13) % 71, nk + 5)
    ks[::29] = -3          # starts before the first key
    ke[5::31] = nk         # ends at the last key
    ks[7], ke[7] = 0, nk   # the whole row
    ks[9], ke[9] = 40, 40  # empty
    return torch.from_numpy(ks.astype(np.int32)), torch.from_numpy(ke.astype(np.int32))


CASES = [(torch.bfloat16, 128), (torch.float16, 64)]


@pytest.mark.parametrize("dtype,d", CASES)
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("ranged", [False, True])
def test_boundaries_at_every_tile_offset(dtype, d, causal, ranged):
    B, H, nq, nk = 1, 2, 300, 300
    q, k, v, do = (normal((B, H, n, d), dtype, 400 + s) for s, n in enumerate((nq, nk, nk, nq)))
    scale = 1.0 / math.sqrt(d)
    kw = dict(scale=scale, causal=causal)
    okw = dict(causal=causal)
    if ranged:
        ks, ke = offset_ranges(nq, nk)
        kw.update(key_start=ks.to(DEV), key_end=ke.to(DEV))
        okw.update(key_start=ks.numpy(), key_end=ke.numpy())
    qd, kd, vd, dod = (t.to(DEV) for t in (q, k, v, do))
    o, lse = fa.fa_fwd(qd, kd, vd, **kw)
    dq, dk, dv = fa.fa_bwd(dod, qd, kd, vd, o, lse, **kw)
    torch.cuda.synchronize()
    what = f"{dtype} d{d} causal={causal} ranged={ranged}"
    o_ref, lse_ref = oracle.attention_forward(np64(q), np64(k), np64(v), scale, **okw)
    assert_fwd_close(np64(o), np64(lse), o_ref, lse_ref, dtype, what)
    want = oracle.attention_backward(np64(q), np64(k), np64(v), np64(do), scale, **okw)
    for name, g, w in zip(("dQ", "dK", "dV"), (dq, dk, dv), want):
        g = np64(g)
        assert np.isfinite(g).all(), f"{what}: non-finite {name}"
        err = float(np.abs(g - w).max())
        assert err <= GRAD_TOL, f"{what}: {name} max err {err:.3e} > {GRAD_TOL}"
