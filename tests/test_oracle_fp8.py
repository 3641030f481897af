"""Pins of the FP8 oracle (``oracle/fp8.py``) against the E4M3 format definition, the
algebra of the Hadamard rotation and brute force. CPU only.

Source of the method: marketmaker.cc blog on Flash Attention, section "FA3: Mekanika
hopper", item 3 (random rotation before block quantisation; lower error than plain FP8
on inputs with outliers).
"""

import itertools

import numpy as np
import pytest
import torch

import oracle
from oracle import fp8 as F
from synth import random_signs, with_outliers

ALL = np.arange(256, dtype=np.uint8)
FINITE = ALL[(ALL & 0x7F) != 0x7F]


# ---- E4M3 codec ---------------------------------------------------------------------
@pytest.mark.parametrize("code,value", [
    (0x00, 0.0), (0x01, 2.0 ** -9), (0x07, 7 * 2.0 ** -9), (0x08, 2.0 ** -6),
    (0x38, 1.0), (0x3C, 1.5), (0x40, 2.0), (0x77, 240.0), (0x7E, 448.0),
    (0xB8, -1.0), (0xFE, -448.0), (0x81, -(2.0 ** -9)),
])
def test_decode_known_values(code, value):
    # sign | exponent (bias 7) | mantissa; exponent 0 is subnormal m * 2^-9
    assert F.e4m3_decode(np.uint8(code)) == value


def test_decode_nan_and_negative_zero():
    assert np.isnan(F.e4m3_decode(np.uint8(0x7F))) and np.isnan(F.e4m3_decode(np.uint8(0xFF)))
    z = F.e4m3_decode(np.uint8(0x80))
    assert z == 0.0 and np.signbit(z)


def test_decode_matches_bitwise_formula():
    for c in FINITE:
        s, e, m = int(c) >> 7, (int(c) >> 3) & 15, int(c) & 7
        v = (m / 8.0) * 2.0 ** -6 if e == 0 else (1 + m / 8.0) * 2.0 ** (e - 7)
        assert F.e4m3_decode(c) == (-v if s else v)


def test_round_trip_every_finite_code():
    assert np.array_equal(F.e4m3_round(F.e4m3_decode(FINITE)), FINITE)


def test_round_is_nearest_by_brute_force():
    x = np.random.default_rng(3).standard_normal(4000) * np.exp2(
        np.random.default_rng(4).uniform(-12, 9, 4000))
    x = np.clip(x, -448, 448)
    vals = F.e4m3_decode(FINITE)
    got = F.e4m3_decode(F.e4m3_round(x))
    best = np.abs(x[:, None] - vals[None, :]).min(axis=1)
    assert np.array_equal(np.abs(got - x), best)


@pytest.mark.parametrize("x,code", [
    (1.0625, 0x38),          # tie between 1.0 (0x38, even) and 1.125 (0x39)
    (1.1875, 0x3A),          # tie between 1.125 and 1.25 (0x3A, even)
    (0.5 * 2.0 ** -9, 0x00),  # tie between 0 and the smallest subnormal
    (1.5 * 2.0 ** -9, 0x02),
    (432.0, 0x7E),           # tie between 416 (0x7D) and 448 (0x7E, even)
    (-1.0625, 0xB8),
    (1e6, 0x7E), (-1e6, 0xFE),  # clamped to +-448
    (-1e-9, 0x80),            # the sign survives rounding to zero
])
def test_round_ties_to_even_and_clamp(x, code):
    assert int(F.e4m3_round(np.float64(x))) == code


def test_relative_error_of_normal_values():
    x = np.exp2(np.random.default_rng(5).uniform(-6, 8.7, 5000))
    err = np.abs(F.e4m3_decode(F.e4m3_round(x)) - x) / x
    assert err.max() <= 2.0 ** -4 + 1e-15


# ---- rotation -------------------------------------------------------------------------
@pytest.mark.parametrize("d", [1, 2, 4, 64, 128])
def test_hadamard_is_orthogonal_with_pm1_entries(d):
    h = F.hadamard(d)
    assert set(np.unique(h)) <= {-1.0, 1.0}
    assert np.array_equal(h @ h.T, d * np.eye(d)) and np.array_equal(h, h.T)


def test_hadamard_small_cases():
    assert np.array_equal(F.hadamard(2), [[1, 1], [1, -1]])
    assert np.array_equal(F.hadamard(4)[3], [1, -1, -1, 1])


def test_rotation_keeps_dot_products_up_to_d():
    rng = np.random.default_rng(6)
    q, k = rng.standard_normal((5, 64)), rng.standard_normal((7, 64))
    s = random_signs(64, 11)
    assert np.allclose(F.rotate(q, s) @ F.rotate(k, s).T, 64 * (q @ k.T), rtol=0, atol=1e-10)


def test_rotation_of_a_signed_hadamard_row_is_one_hot():
    # x = signs * H[j]  ->  x diag(signs) H = H[j] H = d e_j
    d, j = 128, 37
    s = np.array(random_signs(d, 12))
    out = F.rotate((s * F.hadamard(d)[j])[None], s)[0]
    want = np.zeros(d)
    want[j] = d
    assert np.array_equal(out, want)


# ---- block quantisation ---------------------------------------------------------------
def _inputs(shape, seed):
    return with_outliers(shape, torch.bfloat16, seed, 0.01, 10.0).float().double().numpy()


@pytest.mark.parametrize("rot", [False, True])
def test_block_amax_and_codes_by_brute_force(rot):
    B, H, N, d = 2, 2, 150, 64
    x = _inputs((B, H, N, d), 21)
    s = random_signs(d, 22) if rot else None
    codes, amax, scale = F.quantize(x, s)
    assert codes.shape == (B, H, 192, d) and amax.shape == (B, H, 3)
    y = F.rotate(x, s) if rot else x
    for b, h, blk in itertools.product(range(B), range(H), range(3)):
        rows = y[b, h, 64 * blk:64 * blk + 64].astype(np.float32)
        assert amax[b, h, blk] == np.abs(rows).max()
        assert scale[b, h, blk] == np.float32(amax[b, h, blk]) / np.float32(448.0)
        inv = np.float32(448.0) / amax[b, h, blk]
        want = F.e4m3_round((rows * inv).astype(np.float32))
        assert np.array_equal(codes[b, h, 64 * blk:64 * blk + len(rows)], want)
    assert not codes[:, :, N:].any()  # padding rows are zero


def test_dequantised_error_within_half_a_step():
    x = _inputs((1, 3, 256, 128), 23)
    codes, _, scale = F.quantize(x)
    back = F.dequantize(codes, scale)
    step = np.maximum(np.abs(back), 2.0 ** -6 * np.repeat(scale, 64, axis=2)[..., None] * 448)
    assert np.all(np.abs(back - x) <= 2.0 ** -4 * step + 1e-12)


def test_per_head_scale_uses_largest_block():
    x = _inputs((2, 2, 200, 64), 24)
    x[1, 0, 150, 3] = 900.0  # the largest value of head (1, 0), in its last block
    _, amax, scale = F.quantize(x, per_head=True)
    assert np.all(scale[1, 0] == np.float32(900.0) / np.float32(448.0))
    assert np.array_equal(scale[0, 1], np.repeat(amax[0, 1].max() / np.float32(448.0), 4))


def test_zero_block_gives_zero_codes_and_scale():
    x = np.zeros((1, 1, 64, 64))
    codes, amax, scale = F.quantize(x)
    assert not codes.any() and amax[0, 0, 0] == 0 and scale[0, 0, 0] == 0


# ---- V: power-of-two block scales -------------------------------------------------------
def _v_exponent_brute(a):
    # linear scan over every admissible exponent, exact float64 comparisons
    for e in range(-127, 200):
        if float(a) <= 448.0 * 2.0 ** e:
            return e
    raise AssertionError


def test_v_block_exponent_by_brute_force():
    rng = np.random.default_rng(27)
    vals = [np.float32(448.0), np.float32(224.0), np.float32(1.0), np.float32(0.875),
            np.nextafter(np.float32(448.0), np.float32(1e9)),
            np.nextafter(np.float32(448.0), np.float32(0.0)),
            np.float32(448.0 * 2.0 ** -20), np.float32(3.0e38), np.float32(1e-40),
            np.float32(448.0 * 2.0 ** -127), np.float32(448.0 * 2.0 ** -128)]
    vals += list((rng.random(200) * 2.0 ** rng.integers(-60, 60, 200)).astype(np.float32))
    for a in vals:
        assert F.v_block_exponent(a) == _v_exponent_brute(a), a
    assert F.v_block_exponent(0.0) == 0


def test_v_codes_by_brute_force_and_blocks_independent():
    B, H, N, d = 1, 2, 200, 64
    x = _inputs((B, H, N, d), 28)
    codes, amax, scale = F.quantize_v(x)
    assert codes.shape == (B, H, 256, d) and scale.shape == (B, H, 4)
    for h, blk in itertools.product(range(H), range(4)):
        rows = x[0, h, 64 * blk:64 * blk + 64].astype(np.float32)
        e = _v_exponent_brute(np.abs(rows).max())
        assert amax[0, h, blk] == np.abs(rows).max() and scale[0, h, blk] == 2.0 ** e
        want = F.e4m3_round((rows.astype(np.float64) / 2.0 ** e).astype(np.float32))
        assert np.array_equal(codes[0, h, 64 * blk:64 * blk + len(rows)], want)
        top = np.abs(F.e4m3_decode(want)).max()
        assert 224.0 < top <= 448.0  # the block amax lands in the top binade of E4M3
    # a block scaled by 2^5 keeps its codes, its scale grows 32-fold, the others stay
    y = x.copy()
    y[0, 1, 64:128] *= 32.0
    c2, _, s2 = F.quantize_v(y)
    assert np.array_equal(c2, codes)
    assert s2[0, 1, 1] == 32.0 * scale[0, 1, 1]
    assert np.array_equal(np.delete(s2.ravel(), 5), np.delete(scale.ravel(), 5))


def test_v_dequantised_error_within_half_a_step():
    x = _inputs((1, 3, 256, 128), 29)
    codes, _, scale = F.quantize_v(x)
    back = F.dequantize(codes, scale)
    step = np.maximum(np.abs(back), 2.0 ** -6 * np.repeat(scale, 64, axis=2)[..., None])
    assert np.all(np.abs(back - x) <= 2.0 ** -4 * step + 1e-12)


def test_one_hot_rotated_operands_are_exact():
    # rows 7 * signs * H[j] rotate to 7 d e_j = 448 e_j: block scale 1 and code 448, so
    # the quantised operands give exactly the scores of the original inputs
    d, n = 64, 64
    s = np.array(random_signs(d, 25))
    hd = F.hadamard(d)
    rng = np.random.default_rng(26)
    q = (7.0 * s * hd[rng.integers(0, d, n)])[None, None]
    k = (7.0 * s * hd[rng.integers(0, d, n)])[None, None]
    # V: exact E4M3 values with 448 among them, so the block scale is 2^0
    v = np.asarray(F.e4m3_decode(rng.integers(0, 0xFF, (1, 1, n, d)).astype(np.uint8) & 0xF7))
    v[0, 0, 5, 7] = 448.0
    qh, kh, vh, div = F.fp8_attention_operands(q, k, v, s)
    assert div == d
    assert np.array_equal(qh @ kh.transpose(0, 1, 3, 2) / div, q @ k.transpose(0, 1, 3, 2))
    assert np.array_equal(vh, v)


def test_rotation_lowers_error_on_outlier_inputs():
    # the page's claim, on synthetic inputs with outliers (1% of Q and K entries drawn with
    # standard deviation 10): attention on rotated, block-quantised operands is closer to
    # the exact result than on plainly quantised ones (one scale per (b, h))
    B, H, N, d = 1, 2, 256, 128
    q = _inputs((B, H, N, d), 31)
    k = _inputs((B, H, N, d), 32)
    v = torch.randn((B, H, N, d), generator=torch.Generator().manual_seed(33)).double().numpy()
    sc = 1 / np.sqrt(d)
    exact, _ = oracle.attention_forward(q, k, v, sc)

    def rmse(qh, kh, vh, div):
        o, _ = oracle.attention_forward(qh, kh, vh, sc / div)
        return np.sqrt(np.mean((o - exact) ** 2))

    cq, _, sq = F.quantize(q, per_head=True)
    ck, _, sk = F.quantize(k, per_head=True)
    cv, _, sv = F.quantize(v, per_head=True)
    plain = rmse(F.dequantize(cq, sq), F.dequantize(ck, sk), F.dequantize(cv, sv), 1.0)
    rotated = rmse(*F.fp8_attention_operands(q, k, v, random_signs(d, 34)))
    assert rotated < plain / 1.2, (plain, rotated)
