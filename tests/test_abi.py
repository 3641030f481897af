"""The C ABI without a GPU: the library loads, exports every declared entry point,
and rejects invalid arguments before launching anything (no compute calls here)."""

import ctypes
import os
import re

import pytest

import exact_io_aware_flash_amd as fa

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "fa.h")

pytestmark = pytest.mark.skipif(not os.path.exists(fa.lib_path()),
                                reason="libfa.so not built (run __graft_entry__.build())")


def declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(fa_[a-z_]+)\s*\(", src)))


def test_header_declares_the_boundary():
    names = declared_functions()
    for want in ("fa_fwd", "fa_bwd", "fa_bwd_workspace_bytes", "fa_mask_summary",
                 "fa_status_string", "fa_version"):
        assert want in names


def test_library_exports_every_declared_symbol():
    lib = ctypes.CDLL(fa.lib_path())
    for name in declared_functions():
        assert hasattr(lib, name), f"{name} missing from libfa.so"


def test_status_strings_and_version():
    lib = fa.load_library()
    for code in range(0, 12):
        s = fa.fa_status_string(code)
        assert isinstance(s, str) and s
    assert fa.fa_status_string(0) == "ok"
    assert "gfx950" in fa.fa_version()
    assert lib.fa_status_string(999) is not None


def test_workspace_bytes():
    # delta (one float per query row) + key-range summary (4 int32 per 64-row tile) +
    # LSE * log2(e) (one float per query row) + one float per (b, h, 128-key block) for
    # the slope gradient, each rounded up to 256 bytes
    assert (fa.fa_bwd_workspace_bytes(2, 16, 8192, 8192, 128)
            == 2 * (2 * 16 * 8192 * 4) + 2048 + 2 * 16 * 64 * 4)
    assert fa.fa_bwd_workspace_bytes(1, 1, 3, 5, 64) == 1024
    assert fa.fa_bwd_workspace_bytes(0, 1, 3, 5, 64) == 0


# Fake, never-dereferenced device addresses: validation fails before any HIP call.
P = 0x7F0000000000
MIS = P + 8


def fwd(**kw):
    lib = fa.load_library()
    a = dict(q=P, k=P, v=P, o=P, lse=P, B=1, H=1, Nq=16, Nk=16, d=64, scale=0.125, causal=0,
             mb=None, dtype=fa.FA_BF16, stream=None)
    a.update(kw)
    return lib.fa_fwd(a["q"], a["k"], a["v"], a["o"], a["lse"], a["B"], a["H"], a["Nq"],
                      a["Nk"], a["d"], a["scale"], a["causal"], a["mb"], a["dtype"], a["stream"])


@pytest.mark.parametrize("kw,status", [
    (dict(q=None), 1), (dict(o=None), 1),
    (dict(B=0), 2), (dict(H=-1), 2), (dict(Nq=0), 2), (dict(Nk=0), 2),
    (dict(Nq=1 << 30, d=128), 2),
    (dict(dtype=7), 3),
    (dict(d=96), 4), (dict(d=256), 4), (dict(d=0), 4),
    (dict(k=MIS), 6), (dict(o=MIS), 6),
    (dict(scale=0.0), 10), (dict(scale=-1.0), 10), (dict(scale=float("nan")), 10),
    (dict(scale=float("inf")), 10),
])
def test_fwd_rejects_invalid_arguments(kw, status):
    assert fwd(**kw) == status


def test_fwd_rejects_malformed_descriptors():
    d = fa.MaskBiasDesc()
    d.bias_kind = 5
    assert fwd(mb=ctypes.byref(d)) == 5
    d = fa.MaskBiasDesc()
    d.key_start = P
    d.key_end = None
    assert fwd(mb=ctypes.byref(d)) == 5
    d = fa.MaskBiasDesc()
    d.bias_kind = fa.FA_BIAS_DIST_LINEAR
    d.n_slopes = 1
    d.slopes = None
    assert fwd(mb=ctypes.byref(d)) == 1
    arr = (ctypes.c_float * 3)(1, 2, 3)
    d.slopes = ctypes.cast(arr, ctypes.POINTER(ctypes.c_float))
    d.n_slopes = 3
    assert fwd(mb=ctypes.byref(d), H=4) == 5  # neither 1 nor H slopes
    d.n_slopes = 1
    arr[0] = float("nan")
    assert fwd(mb=ctypes.byref(d)) == 10
    d = fa.MaskBiasDesc()
    d.key_start = MIS
    d.key_end = P
    assert fwd(mb=ctypes.byref(d)) == 6


def test_block_mask_descriptor_validation():
    def desc(bq=64, bk=128, sb=0, sh=0):
        d = fa.MaskBiasDesc()
        d.block_mask = P
        d.block_q, d.block_k = bq, bk
        d.mask_stride_b, d.mask_stride_h = sb, sh
        return d
    for bad in (dict(bq=32), dict(bk=100), dict(bq=0), dict(bk=-64), dict(sb=-1), dict(sh=-5)):
        d = desc(**bad)
        assert fwd(mb=ctypes.byref(d)) == 5, bad
    d = desc()
    assert fwd(mb=ctypes.byref(d), dtype=fa.FA_F32, d=96) == 4  # float32 too: shape checks
    assert fwd(mb=ctypes.byref(d), Nk=65536 + 64) == 8    # beyond FA_MAX_SPARSE_N
    assert fwd(mb=ctypes.byref(d), Nq=65536 + 1) == 8
    assert ctypes.sizeof(fa.MaskBiasDesc) == 120  # the C layout of fa_mask_bias_desc


def test_bias_tensor_descriptor_validation():
    def desc(bias=P, sb=0, sh=0, si=16):
        d = fa.MaskBiasDesc()
        d.bias_kind = fa.FA_BIAS_TENSOR
        d.bias = bias
        d.bias_stride_b, d.bias_stride_h, d.bias_stride_i = sb, sh, si
        return d
    assert fwd(mb=ctypes.byref(desc(bias=None))) == 1
    assert fwd(mb=ctypes.byref(desc(bias=P + 2))) == 6   # float32: 4-byte alignment
    for bad in (dict(sb=-1), dict(sh=-16), dict(si=-1)):
        assert fwd(mb=ctypes.byref(desc(**bad))) == 5, bad
    assert fwd(mb=ctypes.byref(desc(si=1 << 24))) == 8  # tile offsets would pass 32 bits
    # a bitmap together with a bias tensor and any summed dbias is accepted (a valid
    # backward stops at the 16-byte workspace: nothing launches)
    d = desc()
    d.block_mask, d.block_q, d.block_k = P, 64, 64
    for bits in (fa.FA_DBIAS_SUM_HEADS, fa.FA_DBIAS_SUM_BATCH | fa.FA_DBIAS_SUM_HEADS,
                 fa.FA_DBIAS_SUM_ROWS):
        d.dbias, d.dbias_reduce = P, bits
        assert bwd(mb=ctypes.byref(d), wsb=16) == 7, bits
    # dbias needs the bias tensor, 4-byte aligned; misaligned bias rejected in the backward
    d = desc()
    d.dbias = P + 2
    assert bwd(mb=ctypes.byref(d)) == 6
    d = fa.MaskBiasDesc()
    d.dbias = P
    assert bwd(mb=ctypes.byref(d)) == 5
    arr = (ctypes.c_float * 1)(0.5)
    d.bias_kind, d.n_slopes = fa.FA_BIAS_DIST_LINEAR, 1
    d.slopes = ctypes.cast(arr, ctypes.POINTER(ctypes.c_float))
    assert bwd(mb=ctypes.byref(d)) == 5
    assert bwd(mb=ctypes.byref(desc(bias=P + 1))) == 6
    # dbias_reduce: known bits only, and only together with dbias (a valid descriptor
    # passes on to the workspace check, which a 16-byte workspace fails: nothing launches)
    for bits, status in ((fa.FA_DBIAS_SUM_BATCH | fa.FA_DBIAS_SUM_ROWS, 7), (7, 7), (8, 5),
                         (-1, 5)):
        d = desc()
        d.dbias, d.dbias_reduce = P, bits
        assert bwd(mb=ctypes.byref(d), wsb=16) == status, bits
    d = desc()
    d.dbias_reduce = fa.FA_DBIAS_SUM_HEADS
    assert bwd(mb=ctypes.byref(d)) == 5


def bwd(**kw):
    lib = fa.load_library()
    a = dict(q=P, k=P, v=P, o=P, lse=P, do=P, dq=P, dk=P, dv=P, gdt=fa.FA_F32, ws=P, wsb=1 << 20,
             B=1, H=1, Nq=16, Nk=16, d=128, scale=0.1, causal=1, mb=None, dtype=fa.FA_BF16,
             stream=None)
    a.update(kw)
    return lib.fa_bwd(a["q"], a["k"], a["v"], a["o"], a["lse"], a["do"], a["dq"], a["dk"],
                      a["dv"], a["gdt"], a["ws"], a["wsb"], a["B"], a["H"], a["Nq"], a["Nk"],
                      a["d"], a["scale"], a["causal"], a["mb"], a["dtype"], a["stream"])


@pytest.mark.parametrize("kw,status", [
    (dict(do=None), 1), (dict(lse=None), 1), (dict(dk=None), 1),
    (dict(gdt=fa.FA_F16), 3),
    (dict(ws=None), 7), (dict(wsb=16), 7),
    (dict(d=32), 4), (dict(Nk=0), 2),
    (dict(dv=MIS), 6), (dict(ws=MIS), 6),
    (dict(scale=0.0), 10),
])
def test_bwd_rejects_invalid_arguments(kw, status):
    assert bwd(**kw) == status


def test_bwd_atomic_dq_phase_validation():
    A = fa.FA_BWD_DQ_ATOMIC
    assert bwd_phases(A) == 10                                   # without the dK/dV pass
    assert bwd_phases(fa.FA_BWD_ALL | A) == 10                   # with the separate dQ pass
    assert bwd_phases(16) == 10
    assert bwd_phases(fa.FA_BWD_DKDV | A, gdt=fa.FA_BF16) == 8   # float32 dq only
    assert bwd_phases(fa.FA_BWD_DKDV | A, dtype=fa.FA_F32) == 8
    d = fa.MaskBiasDesc()
    d.block_mask, d.block_q, d.block_k = P, 64, 64
    assert bwd_phases(fa.FA_BWD_DKDV | A, mb=ctypes.byref(d)) == 8
    # a valid request reaches the workspace check (16 bytes: too small, nothing launches)
    assert bwd_phases(fa.FA_BWD_PREP | fa.FA_BWD_DKDV | A, wsb=16) == 7


def bwd_phases(phases, **kw):
    lib = fa.load_library()
    a = dict(q=P, k=P, v=P, o=P, lse=P, do=P, dq=P, dk=P, dv=P, gdt=fa.FA_F32, ws=P, wsb=1 << 20,
             B=1, H=1, Nq=16, Nk=16, d=128, scale=0.1, causal=1, mb=None, dtype=fa.FA_BF16,
             stream=None)
    a.update(kw)
    return lib.fa_bwd_phases(phases, a["q"], a["k"], a["v"], a["o"], a["lse"], a["do"], a["dq"],
                             a["dk"], a["dv"], a["gdt"], a["ws"], a["wsb"], a["B"], a["H"],
                             a["Nq"], a["Nk"], a["d"], a["scale"], a["causal"], a["mb"],
                             a["dtype"], a["stream"])


@pytest.mark.parametrize("args,status", [
    ((None, P, 10, 10, 4, P, None), 1),
    ((P, P, 0, 10, 4, P, None), 2),
    ((P, P, 10, 10, 0, P, None), 2),
    ((P, P, 10, 10, 2048, P, None), 2),
    ((P, MIS, 10, 10, 4, P, None), 6),
])
def test_mask_summary_rejects_invalid_arguments(args, status):
    assert fa.load_library().fa_mask_summary(*args) == status


def test_python_binding_refuses_cpu_tensors():
    import torch
    q = torch.zeros(1, 1, 4, 64, dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        fa.fa_fwd(q, q, q)


# ---- split-key forward: range plan, workspace size, validation -----------------------

@pytest.mark.parametrize("shape,n_req,n_eff", [
    ((8, 32, 1, 8192, 128), 0, 2),      # 256 units -> 2 ranges of 4096 keys
    ((8, 32, 16, 32768, 128), 0, 2),    # 256 units -> 2 ranges of 16384 keys
    ((1, 32, 1, 32768, 128), 0, 16),    # 32 units -> 16 ranges
    ((1, 1, 1, 8192, 128), 0, 32),      # one unit -> capped at 4 tiles per range
    ((1, 1, 1, 100, 64), 0, 1),         # too short to split
    ((1, 1, 1, 1000, 64), 7, 6),        # 16 tiles, 3 per range -> 6 ranges
    ((1, 1, 1, 1000, 64), 1000, 16),    # at most one range per tile
    ((2, 4, 300, 5000, 64), 3, 3),
])
def test_split_count(shape, n_req, n_eff):
    assert fa.fa_fwd_split_count(*shape, n_req) == n_eff


def test_split_count_rejects_invalid_sizes():
    assert fa.fa_fwd_split_count(1, 1, 1, 1000, 96, 0) == 0
    assert fa.fa_fwd_split_count(1, 1, 0, 1000, 64, 0) == 0
    assert fa.fa_fwd_split_count(1, 1, 1, 1000, 64, -1) == 0


def test_split_workspace_bytes():
    # n * B * H * N_q * d float32 partial outputs + n * B * H * N_q float32 LSEs,
    # each rounded up to 256 bytes; nothing when the effective count is 1
    assert fa.fa_fwd_split_workspace_bytes(8, 32, 1, 8192, 128, 0) == 2 * 256 * 128 * 4 + 2048
    assert fa.fa_fwd_split_workspace_bytes(1, 1, 3, 1000, 64, 7) == 4608 + 256
    assert fa.fa_fwd_split_workspace_bytes(1, 1, 1, 100, 64, 0) == 0


def fwd_split(**kw):
    lib = fa.load_library()
    a = dict(q=P, k=P, v=P, o=P, lse=P, B=1, H=2, Nq=4, Nk=4096, d=128, scale=0.1, causal=0,
             mb=None, dtype=fa.FA_BF16, n=8, ws=P, wsb=1 << 24, stream=None)
    a.update(kw)
    return lib.fa_fwd_split(a["q"], a["k"], a["v"], a["o"], a["lse"], a["B"], a["H"], a["Nq"],
                            a["Nk"], a["d"], a["scale"], a["causal"], a["mb"], a["dtype"],
                            a["n"], a["ws"], a["wsb"], a["stream"])


@pytest.mark.parametrize("kw,status", [
    (dict(n=-1), 10), (dict(q=None), 1), (dict(Nq=0), 2), (dict(d=80), 4),
    (dict(dtype=fa.FA_F32, wsb=1024), 7),  # float32 splits too: stops at the workspace
    (dict(ws=None), 7), (dict(wsb=1024), 7), (dict(ws=MIS), 6), (dict(v=MIS), 6),
    (dict(scale=float("nan")), 10),
    (dict(n=1, q=None), 1),  # effective count 1: validated as fa_fwd
])
def test_fwd_split_rejects_invalid_arguments(kw, status):
    assert fwd_split(**kw) == status


# ---- allocation-free backward: validation before any HIP call --------------------------

def bwd_noalloc(**kw):
    lib = fa.load_library()
    a = dict(q=P, k=P, v=P, o=P, lse=P, do=P, dq=P, dk=P, dv=P, gdt=fa.FA_F32,
             B=1, H=1, Nq=16, Nk=16, d=128, scale=0.1, causal=1, mb=None, dtype=fa.FA_BF16,
             stream=None)
    a.update(kw)
    return lib.fa_bwd_noalloc(a["q"], a["k"], a["v"], a["o"], a["lse"], a["do"], a["dq"],
                              a["dk"], a["dv"], a["gdt"], a["B"], a["H"], a["Nq"], a["Nk"],
                              a["d"], a["scale"], a["causal"], a["mb"], a["dtype"], a["stream"])


@pytest.mark.parametrize("kw,status", [
    (dict(do=None), 1), (dict(lse=None), 1), (dict(dq=None), 1),
    (dict(gdt=fa.FA_F16), 3), (dict(d=32), 4), (dict(Nk=0), 2),
    (dict(dv=MIS), 6), (dict(scale=0.0), 10),
    # the workspace these sizes need exceeds the fixed scratch: rejected, nothing launched
    (dict(B=64, H=64, Nq=8192, Nk=8192), 11),
    (dict(B=1, H=1, Nq=2_200_000, Nk=64, d=64), 11),
])
def test_bwd_noalloc_rejects_invalid_arguments(kw, status):
    assert bwd_noalloc(**kw) == status


def test_bwd_noalloc_scratch_limit_is_the_workspace_size():
    # a problem fits exactly when fa_bwd's workspace for it fits the scratch
    assert fa.fa_bwd_workspace_bytes(2, 16, 8192, 8192, 128) <= fa.FA_NOALLOC_SCRATCH_BYTES
    assert fa.fa_bwd_workspace_bytes(64, 64, 8192, 8192, 128) > fa.FA_NOALLOC_SCRATCH_BYTES
    assert "scratch" in fa.fa_status_string(11)


# ---- forward with tile counters: validation before any HIP call -------------------------

def test_fwd_tile_counts_validation():
    lib = fa.load_library()
    cfg = (ctypes.c_int * 3)()

    def call(counts=P, config=cfg, dtype=fa.FA_BF16, d=128, q=P):
        return lib.fa_fwd_tile_counts(q, P, P, P, P, 1, 1, 64, 64, d, 0.1, 1, None, dtype, None,
                                      counts, config)
    assert call(counts=None) == 1
    assert call(config=None) == 1
    assert call(q=None) == 1
    assert call(counts=P + 4) == 6
    assert call(dtype=fa.FA_F32) == 8  # counted in the 16-bit kernels only
    assert call(d=96) == 4
