"""Seeded synthetic workloads for exact attention (no attention arithmetic here).

Recipe (shared by tests and bench):

* every tensor is drawn with ``torch.Generator('cpu').manual_seed(1000*wid + t)``
  where ``wid`` is the workload id and ``t`` names the tensor: Q=0, K=1, V=2,
  dO=3, key-range mask=9;
* values are fp32 N(0,1) times a per-workload factor, then rounded to the
  workload dtype with round-to-nearest-even (torch's ``.to``), so that the CPU
  oracle (which up-casts the *rounded* values exactly to fp64) and the GPU see
  identical numbers;
* the key-range mask gives every query row ``i`` a half-open key interval
  ``[start_i, end_i)``: rows are grouped in blocks of ``block`` rows; each block
  draws one offset uniformly, each row adds a jitter in ``[0, jitter)``, and
  every interval has the same width.  With width ``N/2`` and 128-row blocks about
  half of the 128x128 tiles of the score matrix are fully masked;
* a bias tensor is float32 N(0, std) of its own (possibly broadcast) shape, with an
  optional seeded fraction of entries set to -inf.
"""

from __future__ import annotations

import dataclasses
from typing import Optional

import torch

T_Q, T_K, T_V, T_DO, T_MASK = 0, 1, 2, 3, 9

_DTYPES = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}


@dataclasses.dataclass(frozen=True)
class Workload:
    """One synthetic attention workload (shapes, dtype and mask recipe)."""

    wid: int
    name: str
    dtype: str
    B: int
    H: int
    N_q: int
    N_k: int
    d: int
    causal: bool = False
    factor: float = 1.0
    bias_slope: Optional[float] = None  # bias(h,i,j) = slope * |i - j|, same slope every head
    key_range: bool = False  # per-row key interval [start_i, end_i)
    backward: bool = False

    @property
    def torch_dtype(self) -> torch.dtype:
        return _DTYPES[self.dtype]

    @property
    def scale(self) -> float:
        return 1.0 / (self.d ** 0.5)

    def scaled(self, **kw) -> "Workload":
        """Same recipe at other sizes (used for small parity cases)."""
        return dataclasses.replace(self, **kw)


# The five workloads: shapes, dtypes and recipes follow the exact-attention
# configurations this library is measured on.
WORKLOADS = {
    1: Workload(1, "fp32 single head B1 H1 N256 d64", "f32", 1, 1, 256, 256, 64),
    2: Workload(2, "bf16 causal fwd B4 H16 N2048 d128", "bf16", 4, 16, 2048, 2048, 128,
                causal=True, factor=0.5),
    3: Workload(3, "fp16 long-sequence fwd B1 H12 N23400 d64", "f16", 1, 12, 23400, 23400, 64),
    4: Workload(4, "bf16 ALiBi-like bias + key-range mask fwd B2 H8 N8192 d128", "bf16",
                2, 8, 8192, 8192, 128, bias_slope=-0.1 / 64, key_range=True),
    5: Workload(5, "bf16 causal fwd+bwd B2 H16 N8192 d128", "bf16", 2, 16, 8192, 8192, 128,
                causal=True, backward=True),
}


def seed_for(wid: int, t: int) -> int:
    return 1000 * wid + t


def normal(shape, dtype: torch.dtype, seed: int, factor: float = 1.0) -> torch.Tensor:
    """fp32 N(0,1)*factor from a seeded CPU generator, RNE-rounded to ``dtype``."""
    g = torch.Generator("cpu").manual_seed(seed)
    x = torch.randn(*shape, dtype=torch.float32, generator=g)
    if factor != 1.0:
        x = x * factor
    return x.to(dtype)


def qkv_inputs(w: Workload, with_dout: Optional[bool] = None):
    """(q, k, v, dout-or-None) CPU tensors in the workload dtype, [B,H,N,d] contiguous."""
    dt = w.torch_dtype
    q = normal((w.B, w.H, w.N_q, w.d), dt, seed_for(w.wid, T_Q), w.factor)
    k = normal((w.B, w.H, w.N_k, w.d), dt, seed_for(w.wid, T_K), w.factor)
    v = normal((w.B, w.H, w.N_k, w.d), dt, seed_for(w.wid, T_V), w.factor)
    want_do = w.backward if with_dout is None else with_dout
    do = normal((w.B, w.H, w.N_q, w.d), dt, seed_for(w.wid, T_DO), w.factor) if want_do else None
    return q, k, v, do


def key_ranges(n_q: int, n_k: int, seed: int, block: int = 128,
               width: Optional[int] = None, jitter: int = 64):
    """Per-row key intervals [start_i, end_i) as int32 CPU tensors of length n_q.

    Rows are grouped in blocks of ``block``; block r draws an offset
    s_r ~ U{0 .. n_k - width - jitter} and row i of that block gets
    start_i = s_r + u_i with u_i ~ U{0 .. jitter-1}; end_i = start_i + width.
    """
    if width is None:
        width = n_k // 2
    g = torch.Generator("cpu").manual_seed(seed)
    n_blocks = (n_q + block - 1) // block
    hi = max(n_k - width - jitter, 0)
    offs = torch.randint(0, hi + 1, (n_blocks,), generator=g, dtype=torch.int64)
    jit = torch.randint(0, jitter, (n_q,), generator=g, dtype=torch.int64)
    start = offs.repeat_interleave(block)[:n_q] + jit
    end = start + width
    return start.to(torch.int32), end.to(torch.int32)


def with_outliers(shape, dtype: torch.dtype, seed: int, frac: float = 1e-3,
                  outlier_std: float = 10.0) -> torch.Tensor:
    """N(0,1) entries of which a random fraction ``frac`` is redrawn from N(0, outlier_std^2),
    RNE-rounded to ``dtype`` (a synthetic stand-in for activations with outliers)."""
    g = torch.Generator("cpu").manual_seed(seed)
    x = torch.randn(*shape, dtype=torch.float32, generator=g)
    pick = torch.rand(*shape, generator=g) < frac
    big = torch.randn(*shape, dtype=torch.float32, generator=g) * outlier_std
    return torch.where(pick, big, x).to(dtype)


def random_signs(d: int, seed: int):
    """d independent fair draws of +1.0 / -1.0 (a list of floats)."""
    g = torch.Generator("cpu").manual_seed(seed)
    return [1.0 if b else -1.0 for b in (torch.rand(d, generator=g) < 0.5).tolist()]


def bias_tensor(shape, seed: int, std: float = 1.0, neg_inf_frac: float = 0.0) -> torch.Tensor:
    """float32 N(0, std) of ``shape`` from a seeded CPU generator; a fraction
    ``neg_inf_frac`` of the entries (drawn from the same generator) is -inf."""
    g = torch.Generator("cpu").manual_seed(seed)
    x = torch.randn(*shape, dtype=torch.float32, generator=g) * std
    if neg_inf_frac > 0:
        x[torch.rand(*shape, generator=g) < neg_inf_frac] = float("-inf")
    return x
