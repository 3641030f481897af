"""Checks against the numeric facts the pages state (tests/golden/page_facts.json)."""

import json
import os

import numpy as np

import oracle
from oracle import attention as A

GOLD = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "page_facts.json")))


def test_score_matrix_size_order_of_magnitude():
    f = GOLD["score_matrix_fp16"]
    nbytes = f["steps"] ** 2 * f["heads"] * f["bytes_per_element"]
    # the page's 12.9 GB is approximate: the exact product is 13.14e9 bytes
    assert abs(nbytes / 1e9 - f["stated_gb"]) / f["stated_gb"] < 0.03


def test_causal_skipping_saves_about_half():
    f = GOLD["causal_tile_skip"]
    n, b = 8192, 128
    cls = oracle.tile_classes(n, n, b, b, causal=True)
    saved = (cls == A.SKIP).mean()
    assert abs(saved - f["stated_fraction_of_work_saved"]) <= 1.0 / (n // b)


def test_io_ratio_in_stated_range():
    # standard path: Theta(N d + N^2) element accesses; tiled: Theta(N^2 d^2 / M)
    f = GOLD["io_ratio_d64"]
    d, m_elems = f["d"], f["sram_bytes"] / 2  # fp16 elements fitting on chip
    n = 8192
    std = n * d + n * n
    tiled = n * n * d * d / m_elems
    ratio = std / tiled
    assert f["stated_ratio_low"] <= ratio <= 2.5 * f["stated_ratio_high"]
    assert np.isfinite(ratio)
