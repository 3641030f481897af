"""FP8 block quantisation with incoherent processing, and attention on quantised operands.

TEST INFRASTRUCTURE ONLY (CPU oracle): imported by ``tests/``, ``__graft_entry__.smoke()``
and the CPU-baseline leg of ``bench.py``; never by the GPU library.

Source: marketmaker.cc blog on Flash Attention ("Apakah Konteks Sehari Penuh ..."),
section "FA3: Mekanika hopper", item 3: FP8 runs at twice the 16-bit rate; plain FP8
attention is spoiled by outliers; the vectors are rotated randomly before *block*
quantisation so that an outlier's magnitude is spread over all coordinates, with a
reported numerical error 2.6x below plain FP8.

Readings (the page names the idea only):

* FP8 format: OCP FP8 E4M3 ("e4m3fn"): 1 sign bit, 4 exponent bits (bias 7), 3 mantissa
  bits; subnormals m * 2^-9; largest finite value 448; no infinities; S.1111.111 is NaN.
  Rounding to nearest, ties to even, after clamping to [-448, 448]; the sign is kept,
  so a negative value that rounds to zero gives -0 (code 0x80).
* Rotation: one random orthogonal matrix applied to Q and K alike, so that
  (Q M)(K M)^T = Q K^T. M = diag(signs) H_d / sqrt(d) with H_d the Sylvester Hadamard
  matrix (entries +-1, H H^T = d I) and signs a caller-drawn +-1 vector (the random
  numbers are an input). The 1/sqrt(d) normalisation is left out of the stored values
  (the block scale absorbs it): the rotated vector is x diag(signs) H_d, and scores of
  rotated operands are divided by d.
* Blocks: 64 consecutive rows (of one (b, h)) by all d columns, with amax = max |value|
  over the block. Q and K: scale = amax / 448. V is not rotated (that would need the
  inverse rotation of O); its block scale is a power of two, 2^e with e the smallest
  integer (at least -127) such that amax <= 448 * 2^e, and its codes are those of
  x * 2^-e. A power of two is the form of block scale that a scaled matrix product
  applies to its operand itself (an E8M0 exponent), so the V scale of each 64-key block
  enters the P V product exactly. Since E4M3 is a floating-point format, a block scale
  that maps the amax anywhere into (224, 448] changes only which of the block's smallest
  values fall below E4M3's normal range.
* Precision of the code decision (a float decides an integer): the rotated value is the
  exact float64 sum, rounded once to float32; amax, 448 / amax and the product with it
  are float32 (IEEE, correctly rounded); the float32 result is clamped and rounded to
  E4M3. For V the product with 2^-e is exact. A block with amax = 0 stores zeros (scale
  0 for Q and K, 2^0 for V).
"""

from __future__ import annotations

import math

import numpy as np

E4M3_MAX = 448.0
QBLOCK = 64  # rows per quantisation block


def e4m3_decode(codes) -> np.ndarray:
    """float64 values of E4M3 codes (uint8); NaN for the two NaN codes."""
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    sign = np.where(c >> 7, -1.0, 1.0)
    e = (c >> 3) & 15
    m = c & 7
    mag = np.where(e == 0, m * 2.0 ** -9, (1.0 + m / 8.0) * np.exp2(e - 7.0))
    mag = np.where((e == 15) & (m == 7), np.nan, mag)
    return sign * mag


def _positive_table():
    codes = np.arange(127, dtype=np.uint8)  # 0x00 .. 0x7e: every non-negative finite value
    return codes, e4m3_decode(codes)


def e4m3_round(x) -> np.ndarray:
    """E4M3 codes of x: clamp to [-448, 448], then round to nearest, ties to even code."""
    x = np.clip(np.asarray(x, dtype=np.float64), -E4M3_MAX, E4M3_MAX)
    codes, vals = _positive_table()
    a = np.abs(x)
    hi = np.clip(np.searchsorted(vals, a, side="left"), 0, len(vals) - 1)  # vals[hi] >= a
    lo = np.clip(hi - 1, 0, len(vals) - 1)
    d_lo = a - vals[lo]
    d_hi = vals[hi] - a
    pick_hi = (d_hi < d_lo) | ((d_hi == d_lo) & (codes[hi] % 2 == 0))
    c = np.where(pick_hi, codes[hi], codes[lo]).astype(np.uint8)
    c = np.where(a == vals[hi], codes[hi], c).astype(np.uint8)  # exact values
    return np.where(np.signbit(x), c | 0x80, c).astype(np.uint8)  # sign kept, also on zero


def hadamard(d: int) -> np.ndarray:
    """Sylvester Hadamard matrix H_d (d a power of two), float64 entries +-1."""
    if d < 1 or d & (d - 1):
        raise ValueError("d must be a power of two")
    h = np.ones((1, 1))
    while h.shape[0] < d:
        h = np.block([[h, h], [h, -h]])
    return h


def rotate(x, signs) -> np.ndarray:
    """x diag(signs) H_d over the last axis, exact in float64 (no 1/sqrt(d))."""
    x = np.asarray(x, dtype=np.float64)
    s = np.asarray(signs, dtype=np.float64)
    return (x * s) @ hadamard(x.shape[-1])


def _pad_rows(x, rows):
    n = x.shape[-2]
    if n == rows:
        return x
    pad = np.zeros(x.shape[:-2] + (rows - n, x.shape[-1]), dtype=x.dtype)
    return np.concatenate([x, pad], axis=-2)


def quantize(x, signs=None, per_head: bool = False):
    """Block-quantise x [B, H, N, d] to E4M3.

    Rows are padded with zeros to a multiple of 64. Returns (codes [B, H, Np, d] uint8,
    amax [B, H, Np/64] float32 of the (rotated) values per 64-row block, scale used per
    block [B, H, Np/64] float32). With per_head the scale of every block of a (b, h) is
    the largest block amax of that (b, h), over 448 (plain FP8 with one scale per head,
    the form the rotated block quantisation is compared against).
    """
    x = np.asarray(x, dtype=np.float64)
    B, H, N, d = x.shape
    n_p = -(-N // QBLOCK) * QBLOCK
    y = rotate(x, signs) if signs is not None else x
    y = _pad_rows(y.astype(np.float32), n_p)  # one rounding of the exact sum
    nb = n_p // QBLOCK
    blocks = y.reshape(B, H, nb, QBLOCK, d)
    amax = np.abs(blocks).max(axis=(3, 4)).astype(np.float32)
    used = amax.max(axis=2, keepdims=True).repeat(nb, axis=2) if per_head else amax
    scale = (used / np.float32(E4M3_MAX)).astype(np.float32)
    with np.errstate(divide="ignore"):
        inv = np.where(used > 0, np.float32(E4M3_MAX) / np.where(used > 0, used, 1),
                       0).astype(np.float32)
    scaled = (blocks * inv[..., None, None]).astype(np.float32)
    codes = e4m3_round(scaled).reshape(B, H, n_p, d)
    return codes, amax, scale


def v_block_exponent(amax: float) -> int:
    """The exponent e of a V block's scale 2^e: the smallest integer e >= -127 with
    amax <= 448 * 2^e; 0 for an all-zero block. Found by exact comparisons in float64."""
    a = float(amax)
    if a == 0.0:
        return 0
    e = math.frexp(a)[1] - 9  # a < 2^(e + 9), and 448 * 2^e = 0.875 * 2^(e + 9)
    while a > math.ldexp(E4M3_MAX, e):
        e += 1
    while e > -127 and a <= math.ldexp(E4M3_MAX, e - 1):
        e -= 1
    return max(e, -127)


def quantize_v(x):
    """Block-quantise V [B, H, N, d] to E4M3 with power-of-two block scales.

    Rows are padded with zeros to a multiple of 64. Returns (codes [B, H, Np, d] uint8,
    amax [B, H, Np/64] float32, scale [B, H, Np/64] float64 = 2^e per block).
    """
    x = np.asarray(x, dtype=np.float64)
    B, H, N, d = x.shape
    n_p = -(-N // QBLOCK) * QBLOCK
    y = _pad_rows(x.astype(np.float32), n_p)
    nb = n_p // QBLOCK
    blocks = y.reshape(B, H, nb, QBLOCK, d)
    amax = np.abs(blocks).max(axis=(3, 4)).astype(np.float32)
    expo = np.vectorize(v_block_exponent, otypes=[np.int64])(amax)
    scale = np.ldexp(1.0, expo)
    scaled = (blocks.astype(np.float64) * np.ldexp(1.0, -expo)[..., None, None]).astype(np.float32)
    codes = e4m3_round(scaled).reshape(B, H, n_p, d)
    return codes, amax, scale


def dequantize(codes, scale) -> np.ndarray:
    """float64 values codes * scale (scale per 64-row block)."""
    v = e4m3_decode(codes)
    B, H, n_p, d = v.shape
    return (v.reshape(B, H, n_p // QBLOCK, QBLOCK, d) *
            np.asarray(scale, dtype=np.float64)[..., None, None]).reshape(B, H, n_p, d)


def fp8_attention_operands(q, k, v, signs=None):
    """The quantised operands of the FP8 forward, dequantised to float64.

    Returns (Qh, Kh, Vh, score_div) with Qh [B,H,N_q,d], Kh and Vh [B,H,N_k,d] (padding
    rows dropped) such that the FP8 path computes attention with scores
    scale * Qh Kh^T / score_div; score_div = d with a rotation (H H^T = d I), else 1.
    """
    n_q, n_k, d = q.shape[2], k.shape[2], q.shape[3]
    cq, _, sq = quantize(q, signs)
    ck, _, sk = quantize(k, signs)
    cv, _, sv = quantize_v(v)
    qh = dequantize(cq, sq)[:, :, :n_q]
    kh = dequantize(ck, sk)[:, :, :n_k]
    vh = dequantize(cv, sv)[:, :, :n_k]
    return qh, kh, vh, float(d) if signs is not None else 1.0
