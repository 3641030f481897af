"""The allocation-free backward (``fa_bwd_noalloc``) against ``fa_bwd`` through the C ABI.

Both run the same kernels on the same inputs, so their gradients must agree bit for bit
(stronger than the 2e-2 parity bar that ``fa_bwd`` itself meets against the oracle). The
scratch array persists between calls on a GPU: two calls in a row, the second with a
smaller problem, then the first problem again, must each equal ``fa_bwd``'s result.
"""

import math

import pytest
import torch

from synth import bias_tensor, key_ranges, normal

pytestmark = pytest.mark.gpu

fa = pytest.importorskip("exact_io_aware_flash_amd")
DEV = "cuda:0"


def _problem(B, H, nq, nk, d, dtype, seed):
    q, k, v, do = (normal((B, H, n, d), dtype, seed + i).to(DEV)
                   for i, n in enumerate((nq, nk, nk, nq)))
    return q, k, v, do


def _compare(B, H, nq, nk, d, dtype, causal, seed, grad_dtype=torch.float32, **extra):
    q, k, v, do = _problem(B, H, nq, nk, d, dtype, seed)
    fwd_kw = {k_: v_ for k_, v_ in extra.items() if k_ not in ("dslopes", "dbias")}
    o, lse = fa.fa_fwd(q, k, v, causal=causal, **fwd_kw)
    want = fa.fa_bwd(do, q, k, v, o, lse, causal=causal, grad_dtype=grad_dtype, **extra)
    want_extra = {n: t.clone() for n, t in extra.items() if n in ("dslopes", "dbias")}
    if "dslopes" in extra:
        extra["dslopes"].fill_(float("nan"))
    if "dbias" in extra:
        extra["dbias"].fill_(float("nan"))
    grads = tuple(torch.full(g.shape, float("nan"), dtype=grad_dtype, device=DEV) for g in want)
    torch.cuda.synchronize()
    before = torch.cuda.memory_allocated()
    got = fa.fa_bwd_noalloc(do, q, k, v, o, lse, grads, causal=causal, **extra)
    torch.cuda.synchronize()
    assert torch.cuda.memory_allocated() == before
    for name, a, b in zip(("dQ", "dK", "dV"), got, want):
        assert torch.equal(a, b), f"{name} differs from fa_bwd"
    for n, t in want_extra.items():
        assert torch.equal(extra[n], t), f"{n} differs from fa_bwd"


def test_noalloc_equals_fa_bwd_on_consecutive_calls():
    # 1) causal bf16 d128 with key ranges, per-head slopes and their gradient (the scratch
    #    holds D, the exponent offsets, the key-range summary and the slope partials)
    B, H, n, d = 2, 4, 1000, 128
    ks, ke = key_ranges(n, n, seed=7001, block=64, width=n // 2, jitter=32)
    big = dict(scale=1.0 / math.sqrt(d), bias_slopes=[-0.02, 0.01, -0.05, 0.03],
               key_start=ks.to(DEV), key_end=ke.to(DEV),
               dslopes=torch.empty(H, dtype=torch.float32, device=DEV))
    _compare(B, H, n, n, d, torch.bfloat16, True, 7000, **big)
    # 2) a smaller problem right after: fp16 d64, non-causal, a bias tensor with dbias,
    #    float32 gradients
    B2, H2, nq, nk, d2 = 1, 2, 300, 257, 64
    bias = bias_tensor((B2, H2, nq, nk), 7011, 1.0, 0.05).to(DEV)
    small = dict(bias=bias, dbias=torch.empty((B2, H2, nq, nk), dtype=torch.float32, device=DEV))
    _compare(B2, H2, nq, nk, d2, torch.float16, False, 7010, **small)
    # 3) the first problem again, with gradients in the input type
    big["dslopes"] = torch.empty(H, dtype=torch.float32, device=DEV)
    _compare(B, H, n, n, d, torch.bfloat16, True, 7000, grad_dtype=torch.bfloat16, **big)


def test_noalloc_full_size_causal_workload():
    # the bf16 causal B2 H16 N8192 d128 backward (2.1 MB of scratch) equals fa_bwd's
    _compare(2, 16, 8192, 8192, 128, torch.bfloat16, True, 7100)


def test_noalloc_rejects_problems_beyond_the_scratch():
    q = torch.zeros((1, 1, 64, 64), dtype=torch.bfloat16, device=DEV)
    lib = fa.load_library()
    st = lib.fa_bwd_noalloc(q.data_ptr(), q.data_ptr(), q.data_ptr(), q.data_ptr(),
                            q.data_ptr(), q.data_ptr(), q.data_ptr(), q.data_ptr(),
                            q.data_ptr(), fa.FA_F32, 64, 64, 8192, 8192, 64, 0.125, 1, None,
                            fa.FA_BF16, None)
    assert st == 11
