"""GPU parity of the backward with dQ accumulated by float32 atomics in the dK/dV pass
(FA_BWD_DQ_ATOMIC), against the float64 oracle and against the deterministic form.

The recomputation backward as on the marketmaker.cc attention page (the section on the
backward pass recomputing rather than storing): the key-outer pass forms dS for its keys
and, besides dK and dV, adds dS K into dQ. dK and dV come from the same arithmetic as in
the deterministic form and must match it bit for bit; dQ differs only in the order of
its float32 additions and meets the same 2e-2 bound against the oracle.
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


def phases_atomic():
    return fa.FA_BWD_PREP | fa.FA_BWD_DKDV | fa.FA_BWD_DQ_ATOMIC


CASES = [
    # dtype, d, causal, nq, nk
    (torch.bfloat16, 128, True, 520, 520),
    (torch.bfloat16, 128, False, 200, 333),
    (torch.float16, 64, True, 333, 200),
    (torch.float16, 128, False, 1, 1),
    (torch.bfloat16, 64, False, 63, 65),
    (torch.bfloat16, 128, True, 3000, 3000),
]


@pytest.mark.parametrize("dtype,d,causal,nq,nk", CASES)
def test_atomic_dq_matches_oracle_and_deterministic_form(dtype, d, causal, nq, nk):
    B, H = 2, 2
    seed = 5200 + nq + 3 * nk + d
    q, k, v, do = (normal((B, H, n, d), dtype, seed + i) for i, n in enumerate((nq, nk, nk, nq)))
    qd, kd, vd, dod = (t.to(DEV) for t in (q, k, v, do))
    scale = 1.0 / math.sqrt(d)
    o, lse = fa.fa_fwd(qd, kd, vd, causal=causal, scale=scale)
    ref = fa.fa_bwd(dod, qd, kd, vd, o, lse, causal=causal, scale=scale)
    grads = tuple(torch.full((B, H, n, d), float("nan"), dtype=torch.float32, device=DEV)
                  for n in (nq, nk, nk))
    got = fa.fa_bwd(dod, qd, kd, vd, o, lse, causal=causal, scale=scale, grads=grads,
                    phases=phases_atomic())
    torch.cuda.synchronize()
    what = f"{dtype} d{d} c{causal} {nq}x{nk}"
    assert torch.equal(got[1], ref[1]) and torch.equal(got[2], ref[2]), what
    assert torch.isfinite(got[0]).all(), what
    if nq * nk <= 600 * 600:
        want = oracle.attention_backward(np64(q), np64(k), np64(v), np64(do), scale,
                                         causal=causal)
        err = float(np.abs(np64(got[0]) - want[0]).max())
        assert err <= GRAD_TOL, f"{what}: dQ err {err:.3e}"
    # against the deterministic dQ: both within float32 reordering of the same terms
    diff = float((got[0] - ref[0]).abs().max())
    assert diff <= 1e-3, f"{what}: |dQ atomic - dQ separate| {diff:.3e}"


@pytest.mark.parametrize("per_head", [False, True])
def test_atomic_dq_with_slope_bias_ranges_and_dslopes(per_head):
    B, H, nq, nk, d = 1, 3, 520, 450, 128
    dtype = torch.bfloat16
    q, k, v, do = (normal((B, H, n, d), dtype, 5300 + i) for i, n in enumerate((nq, nk, nk, nq)))
    ks, ke = key_ranges(nq, nk, seed=5305, block=64, width=nk // 2, jitter=32)
    slopes = [-0.1 / 64, 0.03, -0.02] if per_head else [-0.05]
    scale = 1.0 / math.sqrt(d)
    qd, kd, vd, dod = (t.to(DEV) for t in (q, k, v, do))
    kw = dict(causal=True, scale=scale, bias_slopes=slopes, key_start=ks.to(DEV),
              key_end=ke.to(DEV))
    o, lse = fa.fa_fwd(qd, kd, vd, **kw)
    ds1 = torch.zeros(len(slopes), dtype=torch.float32, device=DEV)
    ds2 = torch.zeros(len(slopes), dtype=torch.float32, device=DEV)
    ref = fa.fa_bwd(dod, qd, kd, vd, o, lse, dslopes=ds1, **kw)
    got = fa.fa_bwd(dod, qd, kd, vd, o, lse, dslopes=ds2, phases=phases_atomic(), **kw)
    torch.cuda.synchronize()
    assert torch.equal(got[1], ref[1]) and torch.equal(got[2], ref[2])
    assert torch.equal(ds1, ds2)
    want = oracle.attention_backward(np64(q), np64(k), np64(v), np64(do), scale, causal=True,
                                     bias_slopes=np.float32(slopes).astype(np.float64),
                                     key_start=ks.numpy(), key_end=ke.numpy())
    err = float(np.abs(np64(got[0]) - want[0]).max())
    assert err <= GRAD_TOL, f"dQ err {err:.3e}"


def test_atomic_dq_full_size_causal_bf16_n8192():
    # the fwd+bwd workload (bf16 causal B2 H16 N8192 d128): dK, dV bit for bit as the
    # deterministic form; dQ against the oracle on two whole heads
    w = WORKLOADS[5]
    q, k, v, do = qkv_inputs(w)
    qd, kd, vd, dod = (t.to(DEV) for t in (q, k, v, do))
    o, lse = fa.fa_fwd(qd, kd, vd, causal=True, scale=w.scale)
    ref = fa.fa_bwd(dod, qd, kd, vd, o, lse, causal=True, scale=w.scale)
    got = fa.fa_bwd(dod, qd, kd, vd, o, lse, causal=True, scale=w.scale, phases=phases_atomic())
    torch.cuda.synchronize()
    assert torch.equal(got[1], ref[1]) and torch.equal(got[2], ref[2])
    assert float((got[0] - ref[0]).abs().max()) <= 1e-3
    for (b, h) in ((0, 3), (1, 15)):
        one = lambda t: np64(t[b:b + 1, h:h + 1])  # noqa: E731
        want = oracle.attention_backward(one(q), one(k), one(v), one(do), w.scale, causal=True,
                                         max_chunk_elems=1 << 25)
        err = float(np.abs(one(got[0]) - want[0]).max())
        assert err <= GRAD_TOL, f"b{b} h{h}: dQ err {err:.3e}"


def test_atomic_dq_rejects_what_it_does_not_cover():
    q = torch.zeros((1, 1, 64, 64), dtype=torch.bfloat16, device=DEV)
    o, lse = fa.fa_fwd(q, q, q)
    with pytest.raises(fa.FaError) as e:  # 16-bit gradients
        fa.fa_bwd(q, q, q, q, o, lse, grad_dtype=torch.bfloat16, phases=phases_atomic())
    assert e.value.status == 8
    with pytest.raises(fa.FaError) as e:  # together with the separate dQ pass
        fa.fa_bwd(q, q, q, q, o, lse, phases=fa.FA_BWD_ALL | fa.FA_BWD_DQ_ATOMIC)
    assert e.value.status == 10
    bias = torch.zeros((1, 1, 64, 64), dtype=torch.float32, device=DEV)
    with pytest.raises(fa.FaError) as e:  # bias tensor
        fa.fa_bwd(q, q, q, q, o, lse, bias=bias, phases=phases_atomic())
    assert e.value.status == 8
