"""Tiles that no query can see are neither loaded nor computed (counted on the GPU).

Blog "Apakah Konteks Sehari Penuh Mengalahkan Konteks Sepuluh Menit?", section "Causal
masking adalah tempat perdagangan mendapat diskon": key tiles entirely in the future of a
query block are never loaded or computed, which removes about half of the work of causal
attention. ``fa_fwd_tile_counts`` runs the forward with counters: key tiles loaded per
workgroup and (wave, tile) score blocks computed. The expected counts come from the
oracle's visibility rule alone (``oracle.visible_mask``, ``oracle.block_visible``) at the
launch's geometry, and for causal masks and overlapping key ranges they equal the number
of tiles the oracle's brute-force classification (``oracle.tile_classes``) does not mark
SKIP: every tile holding a visible key is processed, and no other.
"""

import math

import numpy as np
import pytest
import torch

import oracle
from oracle.attention import SKIP
from synth import WORKLOADS, key_ranges, normal, qkv_inputs, seed_for
from tests.util import assert_fwd_close, np64

pytestmark = pytest.mark.gpu

fa = pytest.importorskip("exact_io_aware_flash_amd")
DEV = "cuda:0"


def span_tiles(vis, rows_blk, bc):
    """Per block of rows_blk rows: tiles from the first to the last visible key (0 if none)."""
    total = 0
    for r0 in range(0, vis.shape[0], rows_blk):
        cols = np.nonzero(vis[r0:r0 + rows_blk].any(axis=0))[0]
        if cols.size:
            total += cols[-1] // bc - cols[0] // bc + 1
    return total


def listed_tiles(vis, rows_blk, bc, wave_rows):
    """Bitmap case: per block of rows_blk rows, tiles that some wave (wave_rows rows) of it
    needs inside that wave's span of visible keys."""
    total = 0
    n_k = vis.shape[1]
    for r0 in range(0, vis.shape[0], rows_blk):
        need = np.zeros((n_k + bc - 1) // bc, dtype=bool)
        for w0 in range(r0, min(vis.shape[0], r0 + rows_blk), wave_rows):
            v = vis[w0:w0 + wave_rows]
            for t in range(need.shape[0]):
                need[t] |= bool(v[:, t * bc:(t + 1) * bc].any())
        total += int(need.sum())
    return total


def expected(n_q, n_k, causal, ks, ke, config, heads, blocks=None):
    rows_wg, rows_wave, bc = config
    rows = np.arange(n_q)
    vis = oracle.visible_mask(n_q, n_k, rows, causal, ks, ke)
    if blocks is not None:
        vis &= oracle.block_visible(rows, n_k, blocks)
        return (heads * listed_tiles(vis, rows_wg, bc, rows_wave),
                heads * listed_tiles(vis, rows_wave, bc, rows_wave))
    return heads * span_tiles(vis, rows_wg, bc), heads * span_tiles(vis, rows_wave, bc)


def not_skipped(n_q, n_k, causal, ks, ke, rows, bc, heads):
    cls = oracle.tile_classes(n_q, n_k, rows, bc, causal, ks, ke)
    return heads * int((cls != SKIP).sum())


def run(w, q, k, v, **kw):
    o, lse, counts, config = fa.fa_fwd_tile_counts(q.to(DEV), k.to(DEV), v.to(DEV), **kw)
    torch.cuda.synchronize()
    return o, lse, [int(x) for x in counts.cpu()], config


@pytest.mark.parametrize("wid", [2, 4, 5])
def test_workloads_skip_exactly_the_invisible_tiles(wid):
    w = WORKLOADS[wid]
    q, k, v, _ = qkv_inputs(w, with_dout=False)
    kw = dict(causal=w.causal, scale=w.scale)
    ks = ke = None
    if w.key_range:
        ks, ke = key_ranges(w.N_q, w.N_k, seed_for(wid, 9), block=128, width=w.N_k // 2, jitter=64)
        kw.update(key_start=ks.to(DEV), key_end=ke.to(DEV))
        ks, ke = ks.numpy(), ke.numpy()
    if w.bias_slope is not None:
        kw.update(bias_slopes=w.bias_slope)
    o, lse, counts, config = run(w, q, k, v, **kw)
    heads = w.B * w.H
    want = expected(w.N_q, w.N_k, w.causal, ks, ke, config, heads)
    assert counts == list(want), (counts, want, config)
    # the same numbers as the tiles the brute-force classification does not skip
    assert counts[0] == not_skipped(w.N_q, w.N_k, w.causal, ks, ke, config[0], config[2], heads)
    assert counts[1] == not_skipped(w.N_q, w.N_k, w.causal, ks, ke, config[1], config[2], heads)
    dense = heads * math.ceil(w.N_q / config[1]) * math.ceil(w.N_k / config[2])
    if w.causal:
        # about half of the dense (wave, tile) blocks (the page's "about half")
        assert 0.45 < counts[1] / dense < 0.56, (counts[1], dense)
    # the counted call computes the forward itself: one sampled head against the oracle
    b, h = w.B - 1, w.H - 1
    one = lambda t: np64(t[b:b + 1, h:h + 1])  # noqa: E731
    rows = np.arange(0, w.N_q, max(1, w.N_q // 64))
    o_ref, l_ref = oracle.attention_forward_rows(
        one(q), one(k), one(v), w.scale, rows, 0, 0, w.causal,
        None if w.bias_slope is None else float(np.float32(w.bias_slope)), ks, ke)
    assert_fwd_close(np64(o[b, h][torch.as_tensor(rows)]), np64(lse[b, h][torch.as_tensor(rows)]),
                     o_ref, l_ref, w.torch_dtype, w.name)


@pytest.mark.parametrize("dtype,d,causal,nq,nk", [
    (torch.bfloat16, 128, True, 300, 300), (torch.float16, 64, True, 520, 257),
    (torch.bfloat16, 128, False, 257, 520), (torch.float16, 64, True, 1000, 1300)])
def test_small_shapes(dtype, d, causal, nq, nk):
    B, H = 2, 3
    q = normal((B, H, nq, d), dtype, 71)
    k = normal((B, H, nk, d), dtype, 72)
    v = normal((B, H, nk, d), dtype, 73)
    o, lse, counts, config = run(None, q, k, v, causal=causal)
    assert counts == list(expected(nq, nk, causal, None, None, config, B * H)), (counts, config)
    assert counts[1] == not_skipped(nq, nk, causal, None, None, config[1], config[2], B * H)
    o_ref, l_ref = oracle.attention_forward(np64(q), np64(k), np64(v), 1 / math.sqrt(d),
                                            causal=causal)
    assert_fwd_close(np64(o), np64(lse), o_ref, l_ref, dtype, "counted small")


def test_block_bitmap_tiles_are_never_loaded():
    B, H, n, d = 1, 4, 2048, 128
    q, k, v = (normal((B, H, n, d), torch.bfloat16, 80 + i) for i in range(3))
    nb = n // 128
    bm = (np.random.default_rng(81).random((H, nb, nb)) < 0.3).astype(np.uint8)
    o, lse, counts, config = run(None, q, k, v, causal=True,
                                 block_mask=(torch.from_numpy(bm).to(DEV), 128, 128))
    want0 = want1 = 0
    for h in range(H):
        e = expected(n, n, True, None, None, config, 1, blocks=(bm[h], 128, 128))
        want0 += e[0]
        want1 += e[1]
    assert counts == [want0, want1], (counts, want0, want1, config)
    dense_causal = not_skipped(n, n, True, None, None, config[1], config[2], B * H)
    assert counts[1] < 0.45 * dense_causal  # density 0.3 of the causal tiles
