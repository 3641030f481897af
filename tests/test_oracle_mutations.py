"""Planted mistakes in the oracle (on the CPU) must be caught by its pins.

Each case patches one plausible mistake into ``oracle.attention`` and checks that
at least one pin of ``tests/test_oracle.py`` fails.  This shows the pins are
strong enough to detect a dropped term, a wrong sign or an off-by-one index.
"""

import numpy as np
import pytest

from oracle import attention as A
import tests.test_oracle as pins


def _orig(name):
    return getattr(A, name)


def mut_scale_dropped(monkeypatch):
    orig = _orig("scores")

    def bad(q_rows, k, scale, *a, **kw):
        return orig(q_rows, k, 1.0, *a, **kw)
    monkeypatch.setattr(A, "scores", bad)


def mut_bias_sign(monkeypatch):
    orig = _orig("distance_bias")
    monkeypatch.setattr(A, "distance_bias", lambda rows, n_k, slope: -orig(rows, n_k, slope))


def mut_causal_off_by_one(monkeypatch):
    orig = _orig("visible_mask")

    def bad(n_q, n_k, rows, causal, ks, ke):
        vis = orig(n_q, n_k, rows, False, ks, ke)
        if causal:
            j = np.arange(n_k)[None, :]
            vis &= j < (np.asarray(rows)[:, None] + (n_k - n_q))
        return vis
    monkeypatch.setattr(A, "visible_mask", bad)


def mut_causal_top_left(monkeypatch):
    orig = _orig("visible_mask")

    def bad(n_q, n_k, rows, causal, ks, ke):
        vis = orig(n_q, n_k, rows, False, ks, ke)
        if causal:
            vis &= np.arange(n_k)[None, :] <= np.asarray(rows)[:, None]
        return vis
    monkeypatch.setattr(A, "visible_mask", bad)


def mut_range_end_inclusive(monkeypatch):
    orig = _orig("visible_mask")

    def bad(n_q, n_k, rows, causal, ks, ke):
        if ks is None:
            return orig(n_q, n_k, rows, causal, ks, ke)
        return orig(n_q, n_k, rows, causal, ks, np.asarray(ke) + 1)
    monkeypatch.setattr(A, "visible_mask", bad)


def mut_softmax_no_normalise(monkeypatch):
    orig = _orig("_two_pass_softmax")

    def bad(s):
        p, m, l = orig(s)
        return p * np.where(l > 0, l, 1.0)[:, None] ** 0.5, m, l
    monkeypatch.setattr(A, "_two_pass_softmax", bad)


def mut_block_sizes_swapped(monkeypatch):
    # rows indexed by block_k and keys by block_q (an IndexError also counts as caught)
    monkeypatch.setattr(A, "block_visible", lambda rows, n_k, blocks: _orig_block_visible(
        rows, n_k, (blocks[0], blocks[2], blocks[1])))


def mut_block_row_off_by_one(monkeypatch):
    def bad(rows, n_k, blocks):
        bm, bq, bk = blocks
        bm = np.asarray(bm)
        r = np.minimum((np.asarray(rows)[:, None] + 1) // bq, bm.shape[0] - 1)
        return bm[r, np.arange(n_k)[None, :] // bk] != 0
    monkeypatch.setattr(A, "block_visible", bad)


def mut_block_bitmap_ignored(monkeypatch):
    monkeypatch.setattr(A, "_blocks_for", lambda bm, b, h: None)


_orig_block_visible = A.block_visible

FWD_PINS = [
    lambda: [pins.test_forward_matches_multiprecision_brute_force(i)
             for i in range(len(pins.CASES))],
    lambda: pins.test_against_torch_float64_reference(True, 0.02, True, 31, 31),
    lambda: pins.test_against_torch_float64_reference(True, None, False, 23, 50),
    lambda: pins.test_bias_only_geometric_series(),
    lambda: pins.test_uniform_scores_mean_of_visible_values(True),
]


@pytest.mark.parametrize("mutation", [
    mut_scale_dropped, mut_bias_sign, mut_causal_off_by_one, mut_causal_top_left,
    mut_range_end_inclusive, mut_softmax_no_normalise,
])
def test_planted_mistake_is_caught(monkeypatch, mutation):
    mutation(monkeypatch)
    caught = 0
    for pin in FWD_PINS:
        try:
            pin()
        except AssertionError:
            caught += 1
    assert caught >= 1, f"no pin caught {mutation.__name__}"


BLOCK_PINS = [
    lambda: pins.test_block_mask_matches_multiprecision_brute_force(False, None),
    lambda: pins.test_block_permutation_equals_independent_problems(),
    lambda: pins.test_block_mask_with_contiguous_rows_equals_key_ranges(True),
]


@pytest.mark.parametrize("mutation", [
    mut_block_sizes_swapped, mut_block_row_off_by_one, mut_block_bitmap_ignored,
])
def test_planted_block_mask_mistake_is_caught(monkeypatch, mutation):
    mutation(monkeypatch)
    caught = 0
    for pin in BLOCK_PINS:
        try:
            pin()
        except (AssertionError, IndexError):
            caught += 1
    assert caught >= 1, f"no pin caught {mutation.__name__}"


# ---- FP8 oracle (oracle/fp8.py) -----------------------------------------------------
from oracle import fp8 as F8  # noqa: E402
import tests.test_oracle_fp8 as fp8_pins  # noqa: E402

_orig_decode, _orig_round, _orig_hadamard = F8.e4m3_decode, F8.e4m3_round, F8.hadamard


def mut_e4m3_bias_8(monkeypatch):
    monkeypatch.setattr(F8, "e4m3_decode", lambda c: _orig_decode(c) / 2.0)


def mut_e4m3_ties_away(monkeypatch):
    def bad(x):
        c = _orig_round(x)
        x = np.clip(np.asarray(x, dtype=np.float64), -448, 448)
        nxt = np.where(c & 0x80, c + 1, c + 1).astype(np.uint8)  # one step up in magnitude
        tie = (c & 0x7F) < 0x7E
        tie &= np.abs(np.abs(x) - np.abs(_orig_decode(c))) == \
            np.abs(np.abs(_orig_decode(nxt)) - np.abs(x))
        return np.where(tie, nxt, c).astype(np.uint8)
    monkeypatch.setattr(F8, "e4m3_round", bad)


def mut_hadamard_no_minus(monkeypatch):
    monkeypatch.setattr(F8, "hadamard", lambda d: np.abs(_orig_hadamard(d)))


def mut_rotation_signs_ignored(monkeypatch):
    monkeypatch.setattr(F8, "rotate", lambda x, s: np.asarray(x, dtype=np.float64) @
                        _orig_hadamard(np.asarray(x).shape[-1]))


_orig_v_exp = F8.v_block_exponent


def mut_v_exponent_one_too_high(monkeypatch):
    monkeypatch.setattr(F8, "v_block_exponent", lambda a: _orig_v_exp(a) + (a != 0))


FP8_PINS = [
    lambda: [fp8_pins.test_decode_known_values(c, v) for c, v in
             [(0x01, 2.0 ** -9), (0x38, 1.0), (0x7E, 448.0)]],
    lambda: [fp8_pins.test_round_ties_to_even_and_clamp(x, c) for x, c in
             [(1.0625, 0x38), (1.1875, 0x3A), (432.0, 0x7E)]],
    lambda: fp8_pins.test_hadamard_is_orthogonal_with_pm1_entries(64),
    lambda: fp8_pins.test_rotation_of_a_signed_hadamard_row_is_one_hot(),
    lambda: fp8_pins.test_block_amax_and_codes_by_brute_force(True),
    lambda: fp8_pins.test_v_block_exponent_by_brute_force(),
    lambda: fp8_pins.test_v_codes_by_brute_force_and_blocks_independent(),
]


@pytest.mark.parametrize("mutation", [
    mut_e4m3_bias_8, mut_e4m3_ties_away, mut_hadamard_no_minus, mut_rotation_signs_ignored,
    mut_v_exponent_one_too_high,
])
def test_planted_fp8_mistake_is_caught(monkeypatch, mutation):
    mutation(monkeypatch)
    caught = 0
    for pin in FP8_PINS:
        try:
            pin()
        except AssertionError:
            caught += 1
    assert caught >= 1, f"no pin caught {mutation.__name__}"


# ---- bias tensor (oracle/attention.py bias_rows, scores) ------------------------------
import tests.test_oracle_bias as bias_pins  # noqa: E402

_orig_bias_rows, _orig_scores = A.bias_rows, A.scores


def mut_tensor_bias_sign(monkeypatch):
    def bad(*a, **kw):
        r = _orig_bias_rows(*a, **kw)
        return None if r is None else -r
    monkeypatch.setattr(A, "bias_rows", bad)


def mut_tensor_bias_scaled(monkeypatch):
    # scores(q_rows, k, scale, rows, n_q, causal, slope, key_start, key_end, blocks, bias)
    def bad(q_rows, k, scale, *a):
        a = list(a)
        if len(a) > 7 and a[7] is not None:
            a[7] = scale * a[7]
        return _orig_scores(q_rows, k, scale, *a)
    monkeypatch.setattr(A, "scores", bad)


def mut_tensor_bias_rows_reversed(monkeypatch):
    def bad(bias, B, H, n_q, n_k, b, h, rows):
        return _orig_bias_rows(bias, B, H, n_q, n_k, b, h, n_q - 1 - np.asarray(rows))
    monkeypatch.setattr(A, "bias_rows", bad)


BIAS_PINS = [
    lambda: bias_pins.test_forward_with_bias_matches_multiprecision_brute_force(False, 5, 7, 0.0),
    lambda: bias_pins.test_row_constant_bias_shifts_lse_only(),
    lambda: bias_pins.test_log2_bias_equals_the_key_taken_twice(),
    lambda: bias_pins.test_dbias_against_torch_autograd_with_broadcast_bias(),
]


@pytest.mark.parametrize("mutation", [
    mut_tensor_bias_sign, mut_tensor_bias_scaled, mut_tensor_bias_rows_reversed,
])
def test_planted_bias_tensor_mistake_is_caught(monkeypatch, mutation):
    mutation(monkeypatch)
    caught = 0
    for pin in BIAS_PINS:
        try:
            pin()
        except AssertionError:
            caught += 1
    assert caught >= 1, f"no pin caught {mutation.__name__}"
