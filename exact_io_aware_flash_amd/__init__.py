"""Exact IO-aware attention for AMD Instinct MI355X (gfx950).

A thin ctypes binding over the C ABI of ``libfa.so`` (declared in ``include/fa.h``).
The Python side only checks tensors and marshals pointers, sizes and the current
HIP stream; every step of the computation runs in the library's HIP kernels.
PyTorch supplies device memory and streams. If the library is not built, every
call raises: there is no CPU or PyTorch fallback.

Function names follow the C entry points: ``fa_fwd``, ``fa_bwd``,
``fa_bwd_workspace_bytes``, ``fa_mask_summary``, ``fa_status_string``, ``fa_version``.
"""

from __future__ import annotations

import ctypes
import math
import os
from typing import Optional, Sequence, Tuple

import torch

__all__ = [
    "FaError", "fa_fwd", "fa_fwd_split", "fa_fwd_split_count", "fa_fwd_split_workspace_bytes",
    "fa_bwd", "fa_bwd_noalloc", "fa_bwd_workspace_bytes", "fa_mask_summary",
    "fa_fwd_tile_counts",
    "FA_NOALLOC_SCRATCH_BYTES",
    "fa_fp8_rows", "fa_fp8_quantize", "fa_fwd_fp8", "fa_attention_fp8",
    "FA_FP8_Q", "FA_FP8_K", "FA_FP8_V",
    "FA_BWD_PREP", "FA_BWD_DKDV", "FA_BWD_DQ", "FA_BWD_ALL", "FA_BWD_DQ_ATOMIC",
    "FA_DBIAS_SUM_BATCH", "FA_DBIAS_SUM_HEADS", "FA_DBIAS_SUM_ROWS",
    "fa_status_string", "fa_version", "lib_path", "load_library",
]

_HERE = os.path.dirname(os.path.abspath(__file__))
# FA_LIBRARY names another build of the library (e.g. one with host-side sanitizers)
_LIB_PATH = os.environ.get("FA_LIBRARY") or os.path.join(_HERE, "libfa.so")
_LIB = None

FA_F32, FA_F16, FA_BF16 = 0, 1, 2
FA_BIAS_NONE, FA_BIAS_DIST_LINEAR, FA_BIAS_TENSOR = 0, 1, 2
FA_MAX_SLOPES = 256
FA_BWD_PREP, FA_BWD_DKDV, FA_BWD_DQ, FA_BWD_ALL = 1, 2, 4, 7
FA_BWD_DQ_ATOMIC = 8  # dQ by float32 atomics inside the dK/dV launch (see include/fa.h)
FA_DBIAS_SUM_BATCH, FA_DBIAS_SUM_HEADS, FA_DBIAS_SUM_ROWS = 1, 2, 4
FA_FP8_Q, FA_FP8_K, FA_FP8_V = 0, 1, 2
FA_NOALLOC_SCRATCH_BYTES = 16 << 20  # include/fa.h
_DT = {torch.float32: FA_F32, torch.float16: FA_F16, torch.bfloat16: FA_BF16}


class FaError(RuntimeError):
    """A non-zero status returned by the C ABI."""

    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: status {status} ({fa_status_string(status)})")


class MaskBiasDesc(ctypes.Structure):
    _fields_ = [
        ("bias_kind", ctypes.c_int32),
        ("n_slopes", ctypes.c_int32),
        ("slopes", ctypes.POINTER(ctypes.c_float)),
        ("key_start", ctypes.c_void_p),
        ("key_end", ctypes.c_void_p),
        ("block_mask", ctypes.c_void_p),
        ("block_q", ctypes.c_int32),
        ("block_k", ctypes.c_int32),
        ("mask_stride_b", ctypes.c_int64),
        ("mask_stride_h", ctypes.c_int64),
        ("dslopes", ctypes.c_void_p),
        ("bias", ctypes.c_void_p),
        ("bias_stride_b", ctypes.c_int64),
        ("bias_stride_h", ctypes.c_int64),
        ("bias_stride_i", ctypes.c_int64),
        ("dbias", ctypes.c_void_p),
        ("dbias_reduce", ctypes.c_int32),
    ]


def lib_path() -> str:
    return _LIB_PATH


def load_library():
    """Load ``libfa.so`` (raises if it has not been built)."""
    global _LIB
    if _LIB is not None:
        return _LIB
    if not os.path.exists(_LIB_PATH):
        raise RuntimeError(
            f"{_LIB_PATH} is missing: build the HIP library first "
            "(python -m exact_io_aware_flash_amd.build)")
    lib = ctypes.CDLL(_LIB_PATH)
    vp, i32, f32 = ctypes.c_void_p, ctypes.c_int, ctypes.c_float
    desc_p = ctypes.POINTER(MaskBiasDesc)
    lib.fa_fwd.argtypes = [vp, vp, vp, vp, vp, i32, i32, i32, i32, i32, f32, i32, desc_p, i32, vp]
    lib.fa_fwd.restype = i32
    lib.fa_fwd_split.argtypes = [vp, vp, vp, vp, vp, i32, i32, i32, i32, i32, f32, i32, desc_p,
                                 i32, i32, vp, ctypes.c_size_t, vp]
    lib.fa_fwd_split.restype = i32
    lib.fa_fwd_split_count.argtypes = [i32, i32, i32, i32, i32, i32]
    lib.fa_fwd_split_count.restype = i32
    lib.fa_fwd_split_workspace_bytes.argtypes = [i32, i32, i32, i32, i32, i32]
    lib.fa_fwd_split_workspace_bytes.restype = ctypes.c_size_t
    lib.fa_bwd_workspace_bytes.argtypes = [i32, i32, i32, i32, i32]
    lib.fa_bwd_workspace_bytes.restype = ctypes.c_size_t
    lib.fa_bwd.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, i32, vp, ctypes.c_size_t,
                           i32, i32, i32, i32, i32, f32, i32, desc_p, i32, vp]
    lib.fa_bwd.restype = i32
    lib.fa_bwd_phases.argtypes = [i32, vp, vp, vp, vp, vp, vp, vp, vp, vp, i32, vp,
                                  ctypes.c_size_t, i32, i32, i32, i32, i32, f32, i32, desc_p,
                                  i32, vp]
    lib.fa_bwd_phases.restype = i32
    lib.fa_fwd_tile_counts.argtypes = [vp, vp, vp, vp, vp, i32, i32, i32, i32, i32, f32, i32,
                                       desc_p, i32, vp, vp, ctypes.POINTER(ctypes.c_int)]
    lib.fa_fwd_tile_counts.restype = i32
    lib.fa_bwd_noalloc.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, i32, i32, i32, i32, i32,
                                   i32, f32, i32, desc_p, i32, vp]
    lib.fa_bwd_noalloc.restype = i32
    lib.fa_mask_summary.argtypes = [vp, vp, i32, i32, i32, vp, vp]
    lib.fa_mask_summary.restype = i32
    lib.fa_fp8_rows.argtypes = [i32]
    lib.fa_fp8_rows.restype = i32
    lib.fa_fp8_quantize.argtypes = [vp, i32, i32, i32, i32, i32, i32, vp, vp, vp, vp]
    lib.fa_fp8_quantize.restype = i32
    lib.fa_fwd_fp8.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, i32, i32, i32, i32, i32, f32,
                               i32, i32, i32, vp]
    lib.fa_fwd_fp8.restype = i32
    lib.fa_status_string.argtypes = [i32]
    lib.fa_status_string.restype = ctypes.c_char_p
    lib.fa_version.argtypes = []
    lib.fa_version.restype = ctypes.c_char_p
    _LIB = lib
    return lib


def fa_status_string(status: int) -> str:
    return load_library().fa_status_string(int(status)).decode()


def fa_version() -> str:
    return load_library().fa_version().decode()


def fa_bwd_workspace_bytes(B: int, H: int, N_q: int, N_k: int, d: int) -> int:
    return int(load_library().fa_bwd_workspace_bytes(B, H, N_q, N_k, d))


def fa_fwd_split_count(B: int, H: int, N_q: int, N_k: int, d: int, n_split: int = 0) -> int:
    return int(load_library().fa_fwd_split_count(B, H, N_q, N_k, d, n_split))


def fa_fwd_split_workspace_bytes(B: int, H: int, N_q: int, N_k: int, d: int,
                                 n_split: int = 0) -> int:
    return int(load_library().fa_fwd_split_workspace_bytes(B, H, N_q, N_k, d, n_split))


def _stream_ptr(stream: Optional[torch.cuda.Stream]) -> int:
    s = stream if stream is not None else torch.cuda.current_stream()
    return int(s.cuda_stream)


def _check_dev(name: str, t: torch.Tensor, dtype=None, shape=None):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{name} has dtype {t.dtype}, expected {dtype}")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")


def _desc(bias_slopes, key_start, key_end, H, N_q, block_mask=None, B=1, N_k=1, dslopes=None,
          bias=None, dbias=None):
    """Build the mask/bias descriptor; returns (desc or None, keepalive).

    ``block_mask``: (bitmap, block_q, block_k) with bitmap a contiguous uint8 device tensor
    [nbq, nbk] (shared), [H, nbq, nbk] (per head) or [B, H, nbq, nbk], where
    nbq = ceil(N_q / block_q) and nbk = ceil(N_k / block_k); a zero byte masks its block.
    ``bias``: float32 device tensor of 4 dimensions that broadcasts to [B, H, N_q, N_k]
    with key stride 1 after broadcasting (a view with zero strides is fine).
    ``dbias``: contiguous float32 device tensor [B or 1, H or 1, N_q or 1, N_k]: receives
    dS summed over each axis of size 1 (the gradient of a bias broadcast over it).
    """
    if (bias_slopes is None and key_start is None and key_end is None and block_mask is None
            and dslopes is None and bias is None and dbias is None):
        return None, None
    d = MaskBiasDesc()
    keep = []
    if block_mask is not None:
        bm, bq, bk = block_mask
        bq, bk = int(bq), int(bk)
        if bq <= 0 or bk <= 0:
            raise ValueError("block sizes must be positive")
        nbq, nbk = (N_q + bq - 1) // bq, (N_k + bk - 1) // bk
        _check_dev("block_mask", bm, torch.uint8)
        if tuple(bm.shape[-2:]) != (nbq, nbk):
            raise ValueError(f"block_mask must end in ({nbq}, {nbk}), got {tuple(bm.shape)}")
        if bm.dim() == 2:
            sb, sh = 0, 0
        elif bm.dim() == 3 and bm.shape[0] == H:
            sb, sh = 0, nbq * nbk
        elif bm.dim() == 4 and tuple(bm.shape[:2]) == (B, H):
            sb, sh = H * nbq * nbk, nbq * nbk
        else:
            raise ValueError("block_mask must be [nbq, nbk], [H, nbq, nbk] or [B, H, nbq, nbk]")
        d.block_mask = bm.data_ptr()
        d.block_q, d.block_k = bq, bk
        d.mask_stride_b, d.mask_stride_h = sb, sh
    d.bias_kind = FA_BIAS_NONE
    d.n_slopes = 1
    d.slopes = None
    if bias_slopes is not None:
        sl = [float(x) for x in (bias_slopes if isinstance(bias_slopes, Sequence)
                                 else [bias_slopes])]
        arr = (ctypes.c_float * len(sl))(*sl)
        keep.append(arr)
        d.bias_kind = FA_BIAS_DIST_LINEAR
        d.n_slopes = len(sl)
        d.slopes = ctypes.cast(arr, ctypes.POINTER(ctypes.c_float))
    if (key_start is None) != (key_end is None):
        raise ValueError("key_start and key_end must be given together")
    if key_start is not None:
        _check_dev("key_start", key_start, torch.int32, (N_q,))
        _check_dev("key_end", key_end, torch.int32, (N_q,))
        d.key_start = key_start.data_ptr()
        d.key_end = key_end.data_ptr()
    if dslopes is not None:
        _check_dev("dslopes", dslopes, torch.float32, (d.n_slopes,))
        d.dslopes = dslopes.data_ptr()
    if bias is not None:
        if bias_slopes is not None:
            raise ValueError("give either bias_slopes or a bias tensor")
        if not isinstance(bias, torch.Tensor) or not bias.is_cuda or bias.dtype != torch.float32:
            raise ValueError("bias must be a float32 device tensor")
        if bias.dim() != 4:
            raise ValueError("bias must have 4 dimensions broadcastable to [B, H, N_q, N_k]")
        view = bias.expand(B, H, N_q, N_k)
        if N_k > 1 and view.stride(3) != 1:
            raise ValueError("bias needs stride 1 along the key axis")
        d.bias_kind = FA_BIAS_TENSOR
        d.bias = view.data_ptr()
        d.bias_stride_b, d.bias_stride_h, d.bias_stride_i = (
            view.stride(0) if B > 1 else 0, view.stride(1) if H > 1 else 0,
            view.stride(2) if N_q > 1 else 0)
    if dbias is not None:
        _check_dev("dbias", dbias, torch.float32)
        shp = tuple(dbias.shape)
        if (len(shp) != 4 or shp[0] not in (1, B) or shp[1] not in (1, H)
                or shp[2] not in (1, N_q) or shp[3] != N_k):
            raise ValueError(f"dbias has shape {shp}, expected [B or 1, H or 1, N_q or 1, N_k] "
                             f"with B={B}, H={H}, N_q={N_q}, N_k={N_k}")
        d.dbias = dbias.data_ptr()
        d.dbias_reduce = ((FA_DBIAS_SUM_BATCH if shp[0] < B else 0)
                          | (FA_DBIAS_SUM_HEADS if shp[1] < H else 0)
                          | (FA_DBIAS_SUM_ROWS if shp[2] < N_q else 0))
    return d, keep


def fa_fwd(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, causal: bool = False,
           scale: Optional[float] = None, bias_slopes=None,
           key_start: Optional[torch.Tensor] = None, key_end: Optional[torch.Tensor] = None,
           out: Optional[torch.Tensor] = None, lse: Optional[torch.Tensor] = None,
           stream: Optional[torch.cuda.Stream] = None,
           block_mask=None, bias: Optional[torch.Tensor] = None) -> Tuple[torch.Tensor, torch.Tensor]:
    """Exact attention forward on the GPU: returns (O [B,H,N_q,d], LSE [B,H,N_q] float32).

    q: [B,H,N_q,d], k/v: [B,H,N_k,d], all of one dtype (float32, float16, bfloat16).
    ``bias_slopes``: float or a list of 1 or H floats, bias = slope * |i - j|.
    ``bias``: float32 tensor broadcastable to [B,H,N_q,N_k], added after scaling.
    ``key_start``/``key_end``: int32 [N_q] device tensors, row i sees keys in [start, end).
    ``block_mask``: (uint8 bitmap, block_q, block_k), see ``_desc``.
    """
    lib = load_library()
    _check_dev("q", q)
    if q.dim() != 4:
        raise ValueError("q must be [B, H, N_q, d]")
    B, H, N_q, d = q.shape
    N_k = k.shape[2]
    if q.dtype not in _DT:
        raise ValueError(f"unsupported dtype {q.dtype}")
    _check_dev("k", k, q.dtype, (B, H, N_k, d))
    _check_dev("v", v, q.dtype, (B, H, N_k, d))
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    if out is None:
        out = torch.empty_like(q)
    _check_dev("out", out, q.dtype, (B, H, N_q, d))
    if lse is None:
        lse = torch.empty((B, H, N_q), dtype=torch.float32, device=q.device)
    _check_dev("lse", lse, torch.float32, (B, H, N_q))
    desc, keep = _desc(bias_slopes, key_start, key_end, H, N_q, block_mask, B, N_k, bias=bias)
    st = lib.fa_fwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), lse.data_ptr(),
                    B, H, N_q, N_k, d, float(scale), 1 if causal else 0,
                    ctypes.byref(desc) if desc is not None else None, _DT[q.dtype],
                    _stream_ptr(stream))
    del keep
    if st != 0:
        raise FaError(st, "fa_fwd")
    return out, lse


def fa_fwd_tile_counts(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, causal: bool = False,
                       scale: Optional[float] = None, bias_slopes=None,
                       key_start: Optional[torch.Tensor] = None,
                       key_end: Optional[torch.Tensor] = None, block_mask=None,
                       bias: Optional[torch.Tensor] = None,
                       stream: Optional[torch.cuda.Stream] = None):
    """The forward with tile counters (``fa_fwd_tile_counts``): returns (O, LSE, counts,
    config) with counts = [key tiles loaded, summed over workgroups; (wave, tile) score
    blocks computed] and config = (query rows per workgroup, per wave, keys per tile)."""
    lib = load_library()
    _check_dev("q", q)
    B, H, N_q, d = q.shape
    N_k = k.shape[2]
    if q.dtype not in _DT:
        raise ValueError(f"unsupported dtype {q.dtype}")
    _check_dev("k", k, q.dtype, (B, H, N_k, d))
    _check_dev("v", v, q.dtype, (B, H, N_k, d))
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    out = torch.empty_like(q)
    lse = torch.empty((B, H, N_q), dtype=torch.float32, device=q.device)
    counts = torch.zeros(2, dtype=torch.int64, device=q.device)
    config = (ctypes.c_int * 3)()
    desc, keep = _desc(bias_slopes, key_start, key_end, H, N_q, block_mask, B, N_k, bias=bias)
    st = lib.fa_fwd_tile_counts(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(),
                                lse.data_ptr(), B, H, N_q, N_k, d, float(scale),
                                1 if causal else 0,
                                ctypes.byref(desc) if desc is not None else None,
                                _DT[q.dtype], _stream_ptr(stream), counts.data_ptr(), config)
    del keep
    if st != 0:
        raise FaError(st, "fa_fwd_tile_counts")
    return out, lse, counts, tuple(config)


def fa_fwd_split(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, causal: bool = False,
                 scale: Optional[float] = None, bias_slopes=None,
                 key_start: Optional[torch.Tensor] = None,
                 key_end: Optional[torch.Tensor] = None, n_split: int = 0,
                 workspace: Optional[torch.Tensor] = None, out: Optional[torch.Tensor] = None,
                 lse: Optional[torch.Tensor] = None,
                 stream: Optional[torch.cuda.Stream] = None,
                 block_mask=None, bias: Optional[torch.Tensor] = None) -> Tuple[torch.Tensor, torch.Tensor]:
    """Split-key forward (``fa_fwd_split``): same arguments and result as :func:`fa_fwd`,
    with the keys of every head cut into ``n_split`` ranges (0: automatic) whose partial
    results are merged on the GPU. ``workspace``: optional uint8 device tensor of at least
    :func:`fa_fwd_split_workspace_bytes` bytes (allocated here when omitted).
    """
    lib = load_library()
    _check_dev("q", q)
    if q.dim() != 4:
        raise ValueError("q must be [B, H, N_q, d]")
    B, H, N_q, d = q.shape
    N_k = k.shape[2]
    if q.dtype not in _DT:
        raise ValueError(f"unsupported dtype {q.dtype}")
    _check_dev("k", k, q.dtype, (B, H, N_k, d))
    _check_dev("v", v, q.dtype, (B, H, N_k, d))
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    if out is None:
        out = torch.empty_like(q)
    _check_dev("out", out, q.dtype, (B, H, N_q, d))
    if lse is None:
        lse = torch.empty((B, H, N_q), dtype=torch.float32, device=q.device)
    _check_dev("lse", lse, torch.float32, (B, H, N_q))
    need = fa_fwd_split_workspace_bytes(B, H, N_q, N_k, d, n_split)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=q.device)
    _check_dev("workspace", workspace, torch.uint8)
    desc, keep = _desc(bias_slopes, key_start, key_end, H, N_q, block_mask, B, N_k, bias=bias)
    st = lib.fa_fwd_split(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(),
                          lse.data_ptr(), B, H, N_q, N_k, d, float(scale), 1 if causal else 0,
                          ctypes.byref(desc) if desc is not None else None, _DT[q.dtype],
                          int(n_split), workspace.data_ptr(), workspace.numel(),
                          _stream_ptr(stream))
    del keep
    if st != 0:
        raise FaError(st, "fa_fwd_split")
    return out, lse


def fa_bwd(dout: torch.Tensor, q: torch.Tensor, k: torch.Tensor, v: torch.Tensor,
           o: torch.Tensor, lse: torch.Tensor, causal: bool = False,
           scale: Optional[float] = None, bias_slopes=None,
           key_start: Optional[torch.Tensor] = None, key_end: Optional[torch.Tensor] = None,
           grad_dtype: torch.dtype = torch.float32, workspace: Optional[torch.Tensor] = None,
           grads=None, phases: int = FA_BWD_ALL, stream: Optional[torch.cuda.Stream] = None,
           block_mask=None, dslopes: Optional[torch.Tensor] = None,
           bias: Optional[torch.Tensor] = None, dbias: Optional[torch.Tensor] = None):
    """Backward by recomputation: returns (dQ, dK, dV) in ``grad_dtype``.

    ``o`` and ``lse`` are the outputs of :func:`fa_fwd` for the same inputs.
    ``dslopes``: optional float32 device tensor of len(bias_slopes) that receives
    dL/dslope (``fa_mask_bias_desc.dslopes``).
    ``bias``: the forward's bias tensor; ``dbias``: optional float32 device tensor
    [B,H,N_q,N_k] that receives the gradient of every biased score, or with size 1 on any
    of the first three axes (e.g. [1,H,N_q,N_k] for a bias shared over the batch,
    [B,1,1,N_k] for a per-key bias), which receives those gradients summed over that axis.
    ``grads``: optional preallocated (dq, dk, dv); ``phases``: subset of FA_BWD_ALL
    (``fa_bwd_phases``), e.g. to run or time the launches separately with one workspace.
    """
    lib = load_library()
    _check_dev("q", q)
    B, H, N_q, d = q.shape
    N_k = k.shape[2]
    _check_dev("k", k, q.dtype, (B, H, N_k, d))
    _check_dev("v", v, q.dtype, (B, H, N_k, d))
    _check_dev("o", o, q.dtype, (B, H, N_q, d))
    _check_dev("dout", dout, q.dtype, (B, H, N_q, d))
    _check_dev("lse", lse, torch.float32, (B, H, N_q))
    if grad_dtype not in (torch.float32, q.dtype):
        raise ValueError("grad_dtype must be float32 or the input dtype")
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    if grads is None:
        dq = torch.empty((B, H, N_q, d), dtype=grad_dtype, device=q.device)
        dk = torch.empty((B, H, N_k, d), dtype=grad_dtype, device=q.device)
        dv = torch.empty((B, H, N_k, d), dtype=grad_dtype, device=q.device)
    else:
        dq, dk, dv = grads
        _check_dev("dq", dq, grad_dtype, (B, H, N_q, d))
        _check_dev("dk", dk, grad_dtype, (B, H, N_k, d))
        _check_dev("dv", dv, grad_dtype, (B, H, N_k, d))
    wsb = fa_bwd_workspace_bytes(B, H, N_q, N_k, d)
    if workspace is None:
        workspace = torch.empty(max(wsb, 16), dtype=torch.uint8, device=q.device)
    desc, keep = _desc(bias_slopes, key_start, key_end, H, N_q, block_mask, B, N_k, dslopes,
                       bias=bias, dbias=dbias)
    st = lib.fa_bwd_phases(int(phases), q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(),
                    dout.data_ptr(), dq.data_ptr(), dk.data_ptr(), dv.data_ptr(),
                    _DT[grad_dtype], workspace.data_ptr(), workspace.numel() * workspace.element_size(),
                    B, H, N_q, N_k, d, float(scale), 1 if causal else 0,
                    ctypes.byref(desc) if desc is not None else None, _DT[q.dtype],
                    _stream_ptr(stream))
    del keep
    if st != 0:
        raise FaError(st, "fa_bwd_phases")
    return dq, dk, dv


def fa_bwd_noalloc(dout: torch.Tensor, q: torch.Tensor, k: torch.Tensor, v: torch.Tensor,
                   o: torch.Tensor, lse: torch.Tensor, grads, causal: bool = False,
                   scale: Optional[float] = None, bias_slopes=None,
                   key_start: Optional[torch.Tensor] = None,
                   key_end: Optional[torch.Tensor] = None,
                   stream: Optional[torch.cuda.Stream] = None, block_mask=None,
                   dslopes: Optional[torch.Tensor] = None, bias: Optional[torch.Tensor] = None,
                   dbias: Optional[torch.Tensor] = None):
    """The allocation-free backward (``fa_bwd_noalloc``): what :func:`fa_bwd` computes, into
    the caller's preallocated ``grads`` = (dq, dk, dv) (float32 or the input dtype), with
    the library's fixed device scratch in place of a workspace. Neither this wrapper nor
    the library allocates device memory. Calls that overlap on one GPU race."""
    lib = load_library()
    _check_dev("q", q)
    B, H, N_q, d = q.shape
    N_k = k.shape[2]
    _check_dev("k", k, q.dtype, (B, H, N_k, d))
    _check_dev("v", v, q.dtype, (B, H, N_k, d))
    _check_dev("o", o, q.dtype, (B, H, N_q, d))
    _check_dev("dout", dout, q.dtype, (B, H, N_q, d))
    _check_dev("lse", lse, torch.float32, (B, H, N_q))
    dq, dk, dv = grads
    grad_dtype = dq.dtype
    if grad_dtype not in (torch.float32, q.dtype):
        raise ValueError("grad dtype must be float32 or the input dtype")
    _check_dev("dq", dq, grad_dtype, (B, H, N_q, d))
    _check_dev("dk", dk, grad_dtype, (B, H, N_k, d))
    _check_dev("dv", dv, grad_dtype, (B, H, N_k, d))
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    desc, keep = _desc(bias_slopes, key_start, key_end, H, N_q, block_mask, B, N_k, dslopes,
                       bias=bias, dbias=dbias)
    st = lib.fa_bwd_noalloc(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(),
                            lse.data_ptr(), dout.data_ptr(), dq.data_ptr(), dk.data_ptr(),
                            dv.data_ptr(), _DT[grad_dtype], B, H, N_q, N_k, d, float(scale),
                            1 if causal else 0, ctypes.byref(desc) if desc is not None else None,
                            _DT[q.dtype], _stream_ptr(stream))
    del keep
    if st != 0:
        raise FaError(st, "fa_bwd_noalloc")
    return dq, dk, dv


def fa_mask_summary(key_start: torch.Tensor, key_end: torch.Tensor, n_k: int, block_rows: int,
                    stream: Optional[torch.cuda.Stream] = None) -> torch.Tensor:
    """Per block of ``block_rows`` query rows: [min start, max start, min end, max end]."""
    lib = load_library()
    (n_q,) = key_start.shape
    _check_dev("key_start", key_start, torch.int32, (n_q,))
    _check_dev("key_end", key_end, torch.int32, (n_q,))
    nb = (n_q + block_rows - 1) // max(block_rows, 1)
    out = torch.empty((max(nb, 1), 4), dtype=torch.int32, device=key_start.device)
    st = lib.fa_mask_summary(key_start.data_ptr(), key_end.data_ptr(), n_q, n_k, block_rows,
                             out.data_ptr(), _stream_ptr(stream))
    if st != 0:
        raise FaError(st, "fa_mask_summary")
    return out[:nb]


def fa_fp8_rows(n: int) -> int:
    """Rows of a quantised tensor with n rows (n rounded up to a multiple of 64)."""
    return int(load_library().fa_fp8_rows(int(n)))


def fa_fp8_quantize(x: torch.Tensor, layout: int, signs=None,
                    stream: Optional[torch.cuda.Stream] = None) -> Tuple[torch.Tensor, torch.Tensor]:
    """Block-quantise x [B,H,N,d] (bf16 or fp16) to E4M3 (``fa_fp8_quantize``).

    Returns (x8 uint8 [B, H, Np, d] in ``layout``'s byte order, amax float32 [B, H, Np/64]),
    Np = fa_fp8_rows(N). ``signs``: sequence of d values +-1 to rotate rows by
    diag(signs) H_d (FA_FP8_Q / FA_FP8_K only).
    """
    lib = load_library()
    _check_dev("x", x)
    if x.dim() != 4 or x.dtype not in (torch.bfloat16, torch.float16):
        raise ValueError("x must be a bf16/fp16 [B, H, N, d] tensor")
    B, H, N, d = x.shape
    n_p = fa_fp8_rows(N)
    x8 = torch.empty((B, H, n_p, d), dtype=torch.uint8, device=x.device)
    amax = torch.empty((B, H, max(n_p // 64, 1)), dtype=torch.float32, device=x.device)
    keep = None
    sp = None
    if signs is not None:
        sl = [float(v) for v in signs]
        if len(sl) != d:
            raise ValueError(f"signs must hold d = {d} values")
        keep = (ctypes.c_float * d)(*sl)
        sp = ctypes.cast(keep, ctypes.c_void_p)
    st = lib.fa_fp8_quantize(x.data_ptr(), B, H, N, d, _DT[x.dtype], int(layout), sp,
                             x8.data_ptr(), amax.data_ptr(), _stream_ptr(stream))
    del keep
    if st != 0:
        raise FaError(st, "fa_fp8_quantize")
    return x8, amax


def fa_fwd_fp8(q8: torch.Tensor, k8: torch.Tensor, v8: torch.Tensor, q_amax: torch.Tensor,
               k_amax: torch.Tensor, v_amax: torch.Tensor, n_q: int, n_k: int,
               causal: bool = False, scale: Optional[float] = None, rotated: bool = False,
               out_dtype: torch.dtype = torch.bfloat16, out: Optional[torch.Tensor] = None,
               lse: Optional[torch.Tensor] = None,
               stream: Optional[torch.cuda.Stream] = None) -> Tuple[torch.Tensor, torch.Tensor]:
    """FP8 forward on operands from :func:`fa_fp8_quantize` (``fa_fwd_fp8``):
    returns (O [B,H,n_q,d] in ``out_dtype``, LSE [B,H,n_q] float32)."""
    lib = load_library()
    B, H, nqp, d = q8.shape
    nkp = fa_fp8_rows(n_k)
    if nqp != fa_fp8_rows(n_q):
        raise ValueError("q8 rows do not match n_q")
    _check_dev("q8", q8, torch.uint8)
    _check_dev("k8", k8, torch.uint8, (B, H, nkp, d))
    _check_dev("v8", v8, torch.uint8, (B, H, nkp, d))
    _check_dev("q_amax", q_amax, torch.float32, (B, H, nqp // 64))
    _check_dev("k_amax", k_amax, torch.float32, (B, H, nkp // 64))
    _check_dev("v_amax", v_amax, torch.float32, (B, H, nkp // 64))
    if out_dtype not in (torch.bfloat16, torch.float16):
        raise ValueError("out_dtype must be bf16 or fp16")
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    if out is None:
        out = torch.empty((B, H, n_q, d), dtype=out_dtype, device=q8.device)
    _check_dev("out", out, out_dtype, (B, H, n_q, d))
    if lse is None:
        lse = torch.empty((B, H, n_q), dtype=torch.float32, device=q8.device)
    _check_dev("lse", lse, torch.float32, (B, H, n_q))
    st = lib.fa_fwd_fp8(q8.data_ptr(), k8.data_ptr(), v8.data_ptr(), q_amax.data_ptr(),
                        k_amax.data_ptr(), v_amax.data_ptr(), out.data_ptr(), lse.data_ptr(),
                        B, H, int(n_q), int(n_k), d, float(scale), 1 if causal else 0,
                        1 if rotated else 0, _DT[out_dtype], _stream_ptr(stream))
    if st != 0:
        raise FaError(st, "fa_fwd_fp8")
    return out, lse


def fa_attention_fp8(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, causal: bool = False,
                     scale: Optional[float] = None, signs=None,
                     stream: Optional[torch.cuda.Stream] = None) -> Tuple[torch.Tensor, torch.Tensor]:
    """Quantise q, k (rotated when ``signs`` is given) and v, then run the FP8 forward;
    O comes back in q's dtype."""
    q8, qa = fa_fp8_quantize(q, FA_FP8_Q, signs, stream)
    k8, ka = fa_fp8_quantize(k, FA_FP8_K, signs, stream)
    v8, va = fa_fp8_quantize(v, FA_FP8_V, None, stream)
    return fa_fwd_fp8(q8, k8, v8, qa, ka, va, q.shape[2], k.shape[2], causal=causal,
                      scale=scale, rotated=signs is not None, out_dtype=q.dtype, stream=stream)
