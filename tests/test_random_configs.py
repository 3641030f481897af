"""Seeded random combinations of every forward/backward option against the float64
oracle: dtype, head dim, ragged N_q != N_k, causal, a generated slope bias or a float32
bias tensor (broadcast over batches and/or heads), per-row key ranges, block bitmaps
(shared, per head, per (b, h)) and the split-key forward. Each case draws its options
from its own seed, so a failure names a reproducible configuration; the fixed cases in
the other parity tests cover each option alone.

Tolerances as everywhere: O within 2e-2 (16-bit) or 1e-5 (float32), LSE within 1e-3
relative, dQ / dK / dV (16-bit inputs, float32 gradients) within 2e-2.
"""

import math

import numpy as np
import pytest
import torch

import oracle
from synth import bias_tensor, key_ranges, normal
from tests.util import GRAD_TOL, assert_fwd_close, np64

pytestmark = pytest.mark.gpu

fa = pytest.importorskip("exact_io_aware_flash_amd")
DEV = "cuda:0"
N_CASES = 120


def draw(i):
    """The options of case i (pure function of i)."""
    r = np.random.default_rng(52000 + i)
    dtype = [torch.bfloat16, torch.float16, torch.float32][int(r.choice(3, p=[0.45, 0.4, 0.15]))]
    c = dict(dtype=dtype, d=int(r.choice([64, 128])), B=int(r.integers(1, 3)),
             H=int(r.integers(1, 4)), nq=int(r.integers(1, 641)), nk=int(r.integers(1, 641)),
             causal=bool(r.random() < 0.5))
    c["bias"] = str(r.choice(["none", "slopes", "tensor"], p=[0.4, 0.3, 0.3]))
    c["bshape"] = int(r.integers(0, 3))  # tensor: [1,H,..], [B,H,..] or [1,1,..]
    c["ranges"] = bool(r.random() < 0.4)
    c["bitmap"] = bool(r.random() < 0.35)
    c["bq"], c["bk"] = int(r.choice([64, 128])), int(r.choice([64, 128, 192]))
    c["layout"] = int(r.integers(0, 3))
    c["split"] = bool(r.random() < 0.3) and dtype != torch.float32 or (dtype == torch.float32 and r.random() < 0.2)
    c["seed"] = 52000 + 97 * i
    return c


@pytest.mark.parametrize("i", range(N_CASES))
def test_random_configuration(i):
    c = draw(i)
    dtype, d, B, H, nq, nk, causal = (c[x] for x in ("dtype", "d", "B", "H", "nq", "nk", "causal"))
    s = c["seed"]
    q = normal((B, H, nq, d), dtype, s)
    k = normal((B, H, nk, d), dtype, s + 1)
    v = normal((B, H, nk, d), dtype, s + 2)
    do = normal((B, H, nq, d), dtype, s + 3)
    scale = 1.0 / math.sqrt(d)
    gpu, ref = dict(causal=causal, scale=scale), dict(causal=causal)
    if c["bias"] == "slopes":
        slopes = [-0.05 + 0.03 * hh for hh in range(H)]
        gpu["bias_slopes"] = slopes
        ref["bias_slopes"] = np.float32(slopes).astype(np.float64)
    elif c["bias"] == "tensor":
        shp = [(1, H, nq, nk), (B, H, nq, nk), (1, 1, nq, nk)][c["bshape"]]
        bt = bias_tensor(shp, s + 4, 1.0, 0.02)
        gpu["bias"] = bt.to(DEV)
        ref["bias"] = bt.numpy()
    if c["ranges"]:
        ks, ke = key_ranges(nq, nk, seed=s + 5, block=64, width=max(nk // 2, 1), jitter=32)
        gpu.update(key_start=ks.to(DEV), key_end=ke.to(DEV))
        ref.update(key_start=ks.numpy(), key_end=ke.numpy())
    if c["bitmap"]:
        bq, bk = c["bq"], c["bk"]
        nbq, nbk = -(-nq // bq), -(-nk // bk)
        shape = [(nbq, nbk), (H, nbq, nbk), (B, H, nbq, nbk)][c["layout"]]
        bm = (np.random.default_rng(s + 6).random(shape) < 0.6).astype(np.uint8)
        gpu["block_mask"] = (torch.from_numpy(bm).to(DEV), bq, bk)
        ref["block_mask"] = (bm, bq, bk)
    what = f"case {i}: {c}"
    qd, kd, vd, dod = (t.to(DEV) for t in (q, k, v, do))

    o, lse = fa.fa_fwd(qd, kd, vd, **gpu)
    torch.cuda.synchronize()
    o_ref, lse_ref = oracle.attention_forward(np64(q), np64(k), np64(v), scale, **ref)
    assert_fwd_close(np64(o), np64(lse), o_ref, lse_ref, dtype, what + " fwd")

    if c["split"]:
        o2, lse2 = fa.fa_fwd_split(qd, kd, vd, n_split=3, **gpu)
        torch.cuda.synchronize()
        assert_fwd_close(np64(o2), np64(lse2), o_ref, lse_ref, dtype, what + " split")

    if dtype == torch.float32:
        return  # float32 gradients have their own per-element bounds (test_bwd_fp32.py)
    dq, dk, dv = fa.fa_bwd(dod, qd, kd, vd, o, lse, **gpu)
    torch.cuda.synchronize()
    want = oracle.attention_backward(np64(q), np64(k), np64(v), np64(do), scale, **ref)
    for name, g, w in zip(("dQ", "dK", "dV"), (dq, dk, dv), want):
        g = np64(g)
        assert np.isfinite(g).all(), f"{what}: non-finite {name}"
        worst = float(np.abs(g - w).max()) if g.size else 0.0
        assert worst <= GRAD_TOL, f"{what}: {name} max err {worst:.3e} > {GRAD_TOL}"
