"""Helpers shared by the GPU parity tests: input staging and the stated tolerances.

Tolerances (exact-attention targets): max |O_gpu - O_ref| <= 1e-5 for float32 inputs
and <= 2e-2 for bf16/fp16 outputs; |LSE_gpu - LSE_ref| / max(|LSE_ref|, 1) <= 1e-3;
gradients max abs error <= 2e-2 (bf16 inputs, float32 gradients).
"""

from __future__ import annotations

import concurrent.futures as cf
import os

import numpy as np
import torch

O_TOL = {torch.float32: 1e-5, torch.float16: 2e-2, torch.bfloat16: 2e-2}
LSE_RTOL = 1e-3
GRAD_TOL = 2e-2


def np64(t: torch.Tensor) -> np.ndarray:
    """Exact up-cast of a (GPU or CPU) tensor to a float64 numpy array."""
    return t.detach().float().cpu().double().numpy()


def lse_rel_err(lse_gpu: np.ndarray, lse_ref: np.ndarray) -> float:
    fin = np.isfinite(lse_ref)
    if not fin.any():
        return 0.0
    return float((np.abs(lse_gpu[fin] - lse_ref[fin]) / np.maximum(np.abs(lse_ref[fin]), 1.0)).max())


def assert_fwd_close(o_gpu, lse_gpu, o_ref, lse_ref, dtype, what=""):
    """O within the dtype tolerance, LSE within 1e-3 relative; empty rows exact."""
    o_gpu = np.asarray(o_gpu, dtype=np.float64)
    lse_gpu = np.asarray(lse_gpu, dtype=np.float64)
    assert o_gpu.shape == o_ref.shape and lse_gpu.shape == lse_ref.shape
    assert np.isfinite(o_gpu).all(), f"{what}: non-finite O"
    empty = ~np.isfinite(lse_ref)
    if empty.any():
        assert np.all(lse_gpu[empty] == -np.inf), f"{what}: empty rows must have LSE=-inf"
        assert np.all(o_gpu[empty] == 0.0), f"{what}: empty rows must have O=0"
    assert np.isfinite(lse_gpu[~empty]).all(), f"{what}: non-finite LSE on a visible row"
    err_o = float(np.abs(o_gpu - o_ref).max()) if o_ref.size else 0.0
    err_l = lse_rel_err(lse_gpu, lse_ref)
    assert err_o <= O_TOL[dtype], f"{what}: max|dO|={err_o:.3e} > {O_TOL[dtype]}"
    assert err_l <= LSE_RTOL, f"{what}: LSE rel err {err_l:.3e} > {LSE_RTOL}"
    return err_o, err_l


def sample_rows(n: int, count: int, seed: int) -> np.ndarray:
    """First, last, tail-tile and random rows (sorted, unique)."""
    rng = np.random.default_rng(seed)
    fixed = [0, 1, n - 1, n - 2, n // 2, (n // 128) * 128, (n // 256) * 256 - 1]
    rows = set(int(r) for r in fixed if 0 <= r < n)
    rows.update(int(x) for x in rng.integers(0, n, size=count))
    return np.array(sorted(rows), dtype=np.int64)


def oracle_workers() -> int:
    """Worker threads for oracle jobs: the host cores this process may run on, at most 16."""
    return max(1, min(16, len(os.sched_getaffinity(0))))


def run_oracle_jobs(fn, jobs):
    """``[fn(j) for j in jobs]`` on a thread pool, BLAS limited to one thread per call.

    NumPy releases the interpreter lock inside BLAS and inside elementwise loops over
    large arrays, so independent oracle calls (one head, or one chunk of rows of a head)
    run side by side on the host cores; the oracle itself is unchanged.
    """
    from threadpoolctl import threadpool_limits

    with threadpool_limits(1):
        with cf.ThreadPoolExecutor(oracle_workers()) as ex:
            return list(ex.map(fn, jobs))
