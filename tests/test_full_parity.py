"""Full-coverage GPU parity on the five synthetic workloads at their full sizes: every row
of every (b, h) head, element by element, against the float64 oracle on the same inputs.

The correctness check of the blog "Apakah Konteks Sehari Penuh Mengalahkan Konteks
Sepuluh Menit?" (section "Pemeriksaan ketepatan, karena 'tepat' melakukan banyak
pekerjaan") runs the fast path and a float64 reference on identical inputs and takes the
largest error over the whole output. Tolerances: O max abs error <= 1e-5 (float32 inputs)
or 2e-2 (bf16 / fp16), LSE relative error <= 1e-3, dQ / dK / dV (float32 gradients of bf16
inputs) max abs error <= 2e-2.

The launches are the ones the library makes for these shapes (the forward's 8-wave form
on the causal N = 8192 workload, the 4-wave form with key ranges, d = 64 with its tail
tile at N = 23400, the three backward launches). The oracle runs per (head, chunk of
rows) or per head on the host cores (``run_oracle_jobs``); the sampled-row tests in
``test_fwd_parity.py`` stay as the fast path.
"""

import functools

import numpy as np
import pytest
import torch

import oracle
from synth import WORKLOADS, key_ranges, qkv_inputs, seed_for
from tests.util import GRAD_TOL, assert_fwd_close, np64, run_oracle_jobs

pytestmark = pytest.mark.gpu

fa = pytest.importorskip("exact_io_aware_flash_amd")
DEV = "cuda:0"
ROW_CHUNK = 1024


def _mask_kw(w):
    """Bias slope and key ranges of a workload: (GPU kwargs, oracle kwargs)."""
    gpu, ref = {}, {}
    if w.bias_slope is not None:
        gpu["bias_slopes"] = w.bias_slope
        ref["bias_slopes"] = float(np.float32(w.bias_slope))  # the float32 value the GPU gets
    if w.key_range:
        ks, ke = key_ranges(w.N_q, w.N_k, seed_for(w.wid, 9), block=128, width=w.N_k // 2,
                            jitter=64)
        gpu.update(key_start=ks.to(DEV), key_end=ke.to(DEV))
        ref.update(key_start=ks.numpy(), key_end=ke.numpy())
    return gpu, ref


@functools.lru_cache(maxsize=1)
def _forward(wid):
    """Inputs (float64 numpy) and the GPU forward (O, LSE as float64 numpy) of a workload."""
    w = WORKLOADS[wid]
    q, k, v, _ = qkv_inputs(w, with_dout=False)
    gpu_kw, _ = _mask_kw(w)
    o, lse = fa.fa_fwd(q.to(DEV), k.to(DEV), v.to(DEV), causal=w.causal, scale=w.scale, **gpu_kw)
    torch.cuda.synchronize()
    return np64(q), np64(k), np64(v), np64(o), np64(lse)


def _check_forward(wid, heads):
    w = WORKLOADS[wid]
    q, k, v, o, lse = _forward(wid)
    _, ref_kw = _mask_kw(w)
    jobs = [(b, h, r0) for (b, h) in heads for r0 in range(0, w.N_q, ROW_CHUNK)]

    def job(j):
        b, h, r0 = j
        rows = np.arange(r0, min(w.N_q, r0 + ROW_CHUNK), dtype=np.int64)
        return oracle.attention_forward_rows(q, k, v, w.scale, rows, b, h, causal=w.causal,
                                             **ref_kw)

    res = run_oracle_jobs(job, jobs)
    worst_o = worst_l = 0.0
    for (b, h) in heads:
        o_ref = np.concatenate([r[0] for j, r in zip(jobs, res) if j[:2] == (b, h)])
        l_ref = np.concatenate([r[1] for j, r in zip(jobs, res) if j[:2] == (b, h)])
        eo, el = assert_fwd_close(o[b, h], lse[b, h], o_ref, l_ref, w.torch_dtype,
                                  f"{w.name} b{b} h{h}, all rows")
        worst_o, worst_l = max(worst_o, eo), max(worst_l, el)
    print(f"{w.name}: {len(heads)} heads, max|dO| {worst_o:.3e}, max LSE rel {worst_l:.3e}")


def _heads(wid):
    w = WORKLOADS[wid]
    return [(b, h) for b in range(w.B) for h in range(w.H)]


def _groups(wid, n):
    hs = _heads(wid)
    return [hs[i::n] for i in range(n)]


def test_full_fp32_single_head_all_rows():
    _check_forward(1, _heads(1))


@pytest.mark.parametrize("group", range(2))
def test_full_causal_bf16_n2048_all_heads(group):
    _check_forward(2, _groups(2, 2)[group])


@pytest.mark.parametrize("group", range(3))
def test_full_long_sequence_fp16_n23400_all_heads(group):
    _check_forward(3, _groups(3, 3)[group])


@pytest.mark.parametrize("group", range(2))
def test_full_bias_key_range_bf16_n8192_all_heads(group):
    _check_forward(4, _groups(4, 2)[group])


@pytest.mark.parametrize("group", range(2))
def test_full_causal_bf16_n8192_forward_all_heads(group):
    _check_forward(5, _groups(5, 2)[group])


@functools.lru_cache(maxsize=1)
def _backward():
    """Inputs and the GPU backward (dQ, dK, dV float32, as float64 numpy) of the causal
    B2 H16 N8192 d128 workload, from the GPU forward's O and LSE."""
    w = WORKLOADS[5]
    q, k, v, do = qkv_inputs(w)
    qd, kd, vd, dod = (t.to(DEV) for t in (q, k, v, do))
    o, lse = fa.fa_fwd(qd, kd, vd, causal=True, scale=w.scale)
    dq, dk, dv = fa.fa_bwd(dod, qd, kd, vd, o, lse, causal=True, scale=w.scale)
    torch.cuda.synchronize()
    return tuple(np64(t) for t in (q, k, v, do, dq, dk, dv))


@pytest.mark.parametrize("group", range(4))
def test_full_causal_bf16_n8192_backward_all_heads(group):
    w = WORKLOADS[5]
    q, k, v, do, dq, dk, dv = _backward()
    heads = _groups(5, 4)[group]

    def job(bh):
        b, h = bh
        one = lambda t: t[b:b + 1, h:h + 1]  # noqa: E731
        return oracle.attention_backward(one(q), one(k), one(v), one(do), w.scale, causal=True)

    worst = {"dQ": 0.0, "dK": 0.0, "dV": 0.0}
    for (b, h), want in zip(heads, run_oracle_jobs(job, heads)):
        for name, got, ref in zip(("dQ", "dK", "dV"), (dq, dk, dv), want):
            g = got[b, h]
            assert np.isfinite(g).all(), f"b{b} h{h}: non-finite {name}"
            err = float(np.abs(g - ref[0, 0]).max())
            assert err <= GRAD_TOL, f"b{b} h{h}: {name} max err {err:.3e} > {GRAD_TOL}"
            worst[name] = max(worst[name], err)
    print(f"{w.name} backward: {len(heads)} heads, max err " +
          ", ".join(f"{n} {e:.3e}" for n, e in worst.items()))
