"""Plain, slow, float64 CPU oracle for exact scaled-dot-product attention.

TEST INFRASTRUCTURE ONLY: imported by ``tests/``, ``__graft_entry__.smoke()``
and the CPU-baseline leg of ``bench.py``; never by the GPU library.

What it computes (the plain definition, materialised, two-pass softmax):

    S = scale * Q K^T + bias          (masked entries = -inf)
    P = softmax(S) row-wise           (pass 1: row max, pass 2: exp / sum)
    O = P V,   LSE = m + ln(l)

Sources (the pages are cited by title and section):

* "Apakah Konteks Sehari Penuh Mengalahkan Konteks Sepuluh Menit? Perhatian
  Kilat dan Pertanyaan Panjang Urutan" (marketmaker.cc blog on Flash Attention),
  section "Mengapa perhatian terikat pada memori": the definition
  softmax(QK^T/sqrt(d_k))V with the materialised N x N score matrix;
  section "Integrasinya delapan baris": the three-line explicit-score version
  (matmul, masked_fill(-inf) for the causal mask, softmax, matmul) and the
  (batch, heads, seq, head_dim) layout;
  section "Pengulangan softmax online": the naive two-pass softmax (max, then
  exponentiate and normalise) that the online recurrence must equal;
  section "Algoritma Flash Attention": the tiled per-query-block loop modelled
  by ``tiled_online_forward``;
  section "Backward pass: menghitung ulang, bukan menyimpan": only O and the
  softmax statistics are kept for the backward pass;
  section "Causal masking ...": keys in the future of a query are never used.
* scifaro.com "related papers: FlashMask: Efficient and Rich Mask Extension of
  FlashAttention" (the abstract on attention with bias): an additive bias matrix
  added to the query-key scores (here either generated, slope * |i - j|, or given
  as a tensor broadcastable to [B, H, N_q, N_k]).
* briefgpt.xyz page for arXiv 2307.08691, FlashAttention abstract (May 2022):
  the tiled method extends to block-sparse attention (here: a per-row key range,
  and a block bitmap); the related abstract (Jun 2023) on a broad class of sparse
  patterns including key and query dropping.

Readings where the pages are silent (each is also listed in the design notes):

* bias is added after scaling and is not multiplied by ``scale``;
  bias(h, i, j) = slopes[h] * |i - j| with absolute row/column indices;
* a bias tensor's -inf entries mask like any other mask (a row whose every
  visible entry is -inf is empty); its gradient is dS, the gradient with respect
  to the biased score, zero where masked;
* a row attends exactly to keys j with start_i <= j < end_i (one interval per
  query row, shared by every batch and head); any integers are allowed, the
  interval is intersected with [0, N_k);
* causal with N_q != N_k is bottom-right aligned: j <= i + N_k - N_q;
* block-sparse mask: the score matrix of a head is cut into blocks of block_q rows
  by block_k keys, and entries of a block whose bitmap byte is zero are masked
  (an entry is visible when every mask in use allows it); the bitmap is given per
  (batch, head), per head, or once for all;
* a row with no visible key has O = 0 and LSE = -inf;
* LSE is the natural log; the backward pass uses the textbook softmax Jacobian
  (the pages only say that P is recomputed from Q, K and the saved statistics).

Parity pins: every function here is pinned in ``tests/test_oracle.py`` against
brute-force multiprecision evaluation, closed forms, invariants, finite
differences and torch's CPU float64 reference routines.  ``row_block_summary``
and ``tile_classes`` are pinned by brute-force recounting.
"""

from __future__ import annotations

from typing import Optional, Sequence

import numpy as np

NEG_INF = -np.inf


def _f64(x) -> np.ndarray:
    return np.asarray(x, dtype=np.float64)


def visible_mask(n_q: int, n_k: int, rows: np.ndarray, causal: bool,
                 key_start: Optional[np.ndarray], key_end: Optional[np.ndarray]) -> np.ndarray:
    """Boolean [len(rows), n_k]: True where query ``rows[r]`` may use key j.

    Causal rule: a key in the future of the query is never used (blog section
    "Causal masking ..."); with N_q != N_k the diagonal is bottom-right aligned.
    Key-range rule: start_i <= j < end_i.
    """
    rows = np.asarray(rows, dtype=np.int64)
    j = np.arange(n_k, dtype=np.int64)[None, :]
    vis = np.ones((rows.shape[0], n_k), dtype=bool)
    if causal:
        vis &= j <= (rows[:, None] + (n_k - n_q))
    if key_start is not None:
        ks = np.asarray(key_start, dtype=np.int64)[rows][:, None]
        ke = np.asarray(key_end, dtype=np.int64)[rows][:, None]
        vis &= (j >= ks) & (j < ke)
    return vis


def block_visible(rows: np.ndarray, n_k: int, blocks) -> np.ndarray:
    """Boolean [len(rows), n_k] of a block-sparse mask for one (b, h).

    ``blocks`` = (bitmap, block_q, block_k) with bitmap [ceil(N_q/block_q),
    ceil(N_k/block_k)]: entry (i, j) lies in block (i // block_q, j // block_k) and is
    visible exactly when that block's byte is non-zero.
    """
    bm, bq, bk = blocks
    bm = np.asarray(bm)
    rows = np.asarray(rows, dtype=np.int64)
    j = np.arange(n_k, dtype=np.int64)
    return bm[rows[:, None] // int(bq), j[None, :] // int(bk)] != 0


def _blocks_for(block_mask, b: int, h: int):
    """The (bitmap, block_q, block_k) of head (b, h) from a [B,H,..], [H,..] or [..] bitmap."""
    if block_mask is None:
        return None
    bm, bq, bk = block_mask
    bm = np.asarray(bm)
    if bm.ndim == 4:
        bm = bm[b, h]
    elif bm.ndim == 3:
        bm = bm[h]
    return bm, bq, bk


def distance_bias(rows: np.ndarray, n_k: int, slope: float) -> np.ndarray:
    """Additive bias slope * |i - j| for the given query rows, float64 [len(rows), n_k]."""
    rows = np.asarray(rows, dtype=np.int64)
    j = np.arange(n_k, dtype=np.int64)
    return float(slope) * np.abs(rows[:, None] - j[None, :]).astype(np.float64)


def bias_rows(bias, B: int, H: int, n_q: int, n_k: int, b: int, h: int,
              rows: np.ndarray) -> Optional[np.ndarray]:
    """Rows of head (b, h) of a bias tensor broadcastable to [B, H, N_q, N_k], float64."""
    if bias is None:
        return None
    full = np.broadcast_to(np.asarray(bias), (B, H, n_q, n_k))
    return _f64(full[b, h][np.asarray(rows, dtype=np.int64)])


def scores(q_rows: np.ndarray, k: np.ndarray, scale: float, rows: np.ndarray, n_q: int,
           causal: bool = False, bias_slope: Optional[float] = None,
           key_start=None, key_end=None, blocks=None,
           bias: Optional[np.ndarray] = None) -> np.ndarray:
    """S for one (b, h) and a set of query rows: scale * q k^T + bias, masked to -inf.

    ``bias``: the rows' entries of a bias tensor, [len(rows), n_k] (see ``bias_rows``).
    """
    s = float(scale) * (_f64(q_rows) @ _f64(k).T)
    n_k = k.shape[0]
    if bias_slope is not None:
        s = s + distance_bias(rows, n_k, bias_slope)
    if bias is not None:
        s = s + bias
    vis = visible_mask(n_q, n_k, rows, causal, key_start, key_end)
    if blocks is not None:
        vis = vis & block_visible(rows, n_k, blocks)
    s[~vis] = NEG_INF
    return s


def _two_pass_softmax(s: np.ndarray):
    """Row softmax of a materialised score block: pass 1 the row max, pass 2 exp and sum.

    Returns (p, m, l).  Rows that are entirely -inf give p = 0, m = -inf, l = 0.
    """
    m = s.max(axis=1)
    m_safe = np.where(np.isfinite(m), m, 0.0)
    e = np.exp(s - m_safe[:, None])
    l = e.sum(axis=1)
    l_safe = np.where(l > 0, l, 1.0)
    p = e / l_safe[:, None]
    return p, m, l


def _slope_for(bias_slopes, h: int):
    if bias_slopes is None:
        return None
    bs = np.atleast_1d(np.asarray(bias_slopes, dtype=np.float64))
    return float(bs[0] if bs.shape[0] == 1 else bs[h])


def _chunks(n: int, n_k: int, max_elems: int):
    step = max(1, min(n, max_elems // max(n_k, 1)))
    for r0 in range(0, n, step):
        yield np.arange(r0, min(n, r0 + step), dtype=np.int64)


def attention_forward_rows(q, k, v, scale: float, rows: Sequence[int], b: int, h: int,
                           causal: bool = False, bias_slopes=None,
                           key_start=None, key_end=None, block_mask=None, bias=None):
    """O and LSE of selected query rows of one (b, h): ([len(rows), d], [len(rows)])."""
    rows = np.asarray(rows, dtype=np.int64)
    B, H, n_q = q.shape[:3]
    n_k = k.shape[2]
    s = scores(_f64(q[b, h][rows]), _f64(k[b, h]), scale, rows, n_q, causal,
               _slope_for(bias_slopes, h), key_start, key_end, _blocks_for(block_mask, b, h),
               bias_rows(bias, B, H, n_q, n_k, b, h, rows))
    p, m, l = _two_pass_softmax(s)
    o = p @ _f64(v[b, h])
    lse = np.where(l > 0, m + np.log(np.where(l > 0, l, 1.0)), NEG_INF)
    return o, lse


def attention_forward(q, k, v, scale: float, causal: bool = False, bias_slopes=None,
                      key_start=None, key_end=None, max_chunk_elems: int = 1 << 24,
                      block_mask=None, bias=None):
    """Full forward: O [B,H,N_q,d] float64 and LSE [B,H,N_q] float64.

    Inputs are [B,H,N,d] arrays (any float dtype; up-cast exactly to float64).
    ``bias``: optional array broadcastable to [B,H,N_q,N_k], added after scaling.
    Memory stays bounded by processing one (b, h, row-chunk) at a time.
    """
    B, H, n_q, d = q.shape
    n_k = k.shape[2]
    o = np.zeros((B, H, n_q, d), dtype=np.float64)
    lse = np.full((B, H, n_q), NEG_INF, dtype=np.float64)
    for b in range(B):
        for h in range(H):
            for rows in _chunks(n_q, n_k, max_chunk_elems):
                o[b, h, rows], lse[b, h, rows] = attention_forward_rows(
                    q, k, v, scale, rows, b, h, causal, bias_slopes, key_start, key_end,
                    block_mask, bias)
    return o, lse


def attention_probabilities(q, k, scale: float, b: int = 0, h: int = 0, causal: bool = False,
                            bias_slopes=None, key_start=None, key_end=None,
                            block_mask=None, bias=None) -> np.ndarray:
    """The full probability matrix P [N_q, N_k] of one (b, h) (small inputs only)."""
    B, H, n_q = q.shape[:3]
    rows = np.arange(n_q, dtype=np.int64)
    s = scores(_f64(q[b, h]), _f64(k[b, h]), scale, rows, n_q, causal,
               _slope_for(bias_slopes, h), key_start, key_end, _blocks_for(block_mask, b, h),
               bias_rows(bias, B, H, n_q, k.shape[2], b, h, rows))
    return _two_pass_softmax(s)[0]


def attention_backward(q, k, v, dout, scale: float, causal: bool = False, bias_slopes=None,
                       key_start=None, key_end=None, max_chunk_elems: int = 1 << 24,
                       block_mask=None, return_dslopes: bool = False, bias=None,
                       return_dbias: bool = False):
    """Analytic float64 gradients (dQ, dK, dV) of L = sum(O * dO), each [B,H,N,d].

    Textbook softmax Jacobian with P recomputed from Q and K:
        dV = P^T dO,  dP = dO V^T,  D_i = sum_j P_ij dP_ij,
        dS = P o (dP - D),  dQ = scale * dS K,  dK = scale * dS^T Q.
    No gradient flows to the mask. With return_dslopes (and bias_slopes given) a fourth
    result is dL/dslope: the bias slope_h |i - j| enters S additively, so
        dL/dslope_h = sum_{b, i, j} dS_{b,h,i,j} |i - j|,
    one value per head, or one in all (summed over heads) for a single shared slope.
    With return_dbias (a bias tensor enters S additively, entry by entry) the last result
    is dS itself, [B, H, N_q, N_k] (zero where masked).
    """
    B, H, n_q, d = q.shape
    n_k = k.shape[2]
    dq = np.zeros((B, H, n_q, d), dtype=np.float64)
    dk = np.zeros((B, H, n_k, d), dtype=np.float64)
    dv = np.zeros((B, H, n_k, d), dtype=np.float64)
    dslope = np.zeros(H, dtype=np.float64)
    dbias = np.zeros((B, H, n_q, n_k), dtype=np.float64) if return_dbias else None
    for b in range(B):
        for h in range(H):
            kb, vb = _f64(k[b, h]), _f64(v[b, h])
            for rows in _chunks(n_q, n_k, max_chunk_elems):
                qr, dor = _f64(q[b, h][rows]), _f64(dout[b, h][rows])
                s = scores(qr, kb, scale, rows, n_q, causal, _slope_for(bias_slopes, h),
                           key_start, key_end, _blocks_for(block_mask, b, h),
                           bias_rows(bias, B, H, n_q, n_k, b, h, rows))
                p, _, _ = _two_pass_softmax(s)
                dv[b, h] += p.T @ dor
                dp = dor @ vb.T
                dsum = (p * dp).sum(axis=1)
                ds = p * (dp - dsum[:, None])
                dq[b, h, rows] = float(scale) * (ds @ kb)
                dk[b, h] += float(scale) * (ds.T @ qr)
                if return_dslopes:
                    dslope[h] += float((ds * distance_bias(rows, n_k, 1.0)).sum())
                if return_dbias:
                    dbias[b, h, rows] = ds
    out = [dq, dk, dv]
    if return_dslopes:
        if bias_slopes is None:
            raise ValueError("return_dslopes needs bias_slopes")
        shared = np.atleast_1d(np.asarray(bias_slopes)).shape[0] == 1
        out.append(dslope.sum(keepdims=True) if shared else dslope)
    if return_dbias:
        out.append(dbias)
    return tuple(out)


def tiled_online_forward(q, k, v, scale: float, br: int, bc: int, causal: bool = False,
                         bias_slopes=None, key_start=None, key_end=None, block_mask=None,
                         bias=None):
    """The pages' tiled loop in float64, as a model of the recurrence the GPU runs.

    Blog section "Algoritma Flash Attention": Q is cut into ceil(N/B_r) row
    blocks, K and V into ceil(N/B_c) column blocks; for each query block the
    running max m, running sum l and output accumulator are updated block by
    block.  Section "Pengulangan softmax online" (its display equations are
    missing from the page; the recurrence is rebuilt from the loop): when a block
    raises the running max, the earlier sum and accumulator are rescaled by
    exp(m_old - m_new).  Section "FA2: paralelisme" item 1: the division by l is
    deferred to the end of the inner loop.  Block-level max/sum/exp are taken on
    the whole tile, fully masked tiles are skipped (section "Causal masking ...").
    """
    B, H, n_q, d = q.shape
    n_k = k.shape[2]
    o = np.zeros((B, H, n_q, d), dtype=np.float64)
    lse = np.full((B, H, n_q), NEG_INF, dtype=np.float64)
    for b in range(B):
        for h in range(H):
            slope = _slope_for(bias_slopes, h)
            blocks = _blocks_for(block_mask, b, h)
            for r0 in range(0, n_q, br):
                rows = np.arange(r0, min(n_q, r0 + br), dtype=np.int64)
                qi = _f64(q[b, h][rows])
                acc = np.zeros((rows.shape[0], d))
                m = np.full(rows.shape[0], NEG_INF)
                l = np.zeros(rows.shape[0])
                for c0 in range(0, n_k, bc):
                    cols = np.arange(c0, min(n_k, c0 + bc), dtype=np.int64)
                    s = float(scale) * (qi @ _f64(k[b, h][cols]).T)
                    if slope is not None:
                        s = s + slope * np.abs(rows[:, None] - cols[None, :]).astype(np.float64)
                    if bias is not None:
                        s = s + bias_rows(bias, B, H, n_q, n_k, b, h, rows)[:, cols]
                    vis = visible_mask(n_q, n_k, rows, causal, key_start, key_end)
                    if blocks is not None:
                        vis = vis & block_visible(rows, n_k, blocks)
                    vis = vis[:, cols]
                    if not vis.any():
                        continue  # fully masked tile: never loaded, contributes nothing
                    s[~vis] = NEG_INF
                    m_tile = s.max(axis=1)
                    m_new = np.maximum(m, m_tile)
                    base = np.where(np.isfinite(m_new), m_new, 0.0)
                    alpha = np.exp(m - base)  # exp(-inf) = 0 on the first visible block
                    p = np.exp(s - base[:, None])
                    l = alpha * l + p.sum(axis=1)
                    acc = alpha[:, None] * acc + p @ _f64(v[b, h][cols])
                    m = m_new
                ok = l > 0
                o[b, h, rows[ok]] = acc[ok] / l[ok, None]
                lse[b, h, rows[ok]] = m[ok] + np.log(l[ok])
    return o, lse


def row_block_summary(key_start, key_end, n_k: int, block: int) -> np.ndarray:
    """Per block of ``block`` query rows: [min start, max start, min end, max end].

    Intervals are first intersected with [0, n_k] (start and end clamped), which
    does not change the set of visible keys.  Int64 array [ceil(N_q/block), 4].
    """
    ks = np.clip(np.asarray(key_start, dtype=np.int64), 0, n_k)
    ke = np.clip(np.asarray(key_end, dtype=np.int64), 0, n_k)
    n_q = ks.shape[0]
    out = np.zeros(((n_q + block - 1) // block, 4), dtype=np.int64)
    for r in range(out.shape[0]):
        sl = slice(r * block, min(n_q, (r + 1) * block))
        out[r] = (ks[sl].min(), ks[sl].max(), ke[sl].min(), ke[sl].max())
    return out


SKIP, PARTIAL, FULL = 0, 1, 2


def tile_classes(n_q: int, n_k: int, br: int, bc: int, causal: bool = False,
                 key_start=None, key_end=None, blocks=None) -> np.ndarray:
    """Brute-force class of every (row block, column block) tile of the score matrix.

    SKIP = no visible entry, FULL = every entry visible, PARTIAL otherwise.
    (Fully masked tiles are the ones the method never loads or computes.)
    """
    t_r, t_c = (n_q + br - 1) // br, (n_k + bc - 1) // bc
    out = np.zeros((t_r, t_c), dtype=np.int64)
    for r in range(t_r):
        rows = np.arange(r * br, min(n_q, (r + 1) * br), dtype=np.int64)
        vis = visible_mask(n_q, n_k, rows, causal, key_start, key_end)
        if blocks is not None:
            vis = vis & block_visible(rows, n_k, blocks)
        for c in range(t_c):
            blk = vis[:, c * bc:min(n_k, (c + 1) * bc)]
            out[r, c] = FULL if blk.all() else (PARTIAL if blk.any() else SKIP)
    return out

