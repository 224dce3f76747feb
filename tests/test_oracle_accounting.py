"""Pins for oracle.accounting: brute-force mask counts and the pages' printed figures."""

import json
import os

import numpy as np
import pytest

from oracle.accounting import (
    hybrid_kv_ratio,
    hybrid_prefill_pair_ratio,
    kv_rows,
    visible_keys,
    visible_pairs,
)
from oracle.attention import visible_mask


@pytest.mark.parametrize("kind,window", [("swa", 4), ("swa", 128), ("full", 0)])
def test_visible_pairs_equal_mask_count(kind, window):
    for hist, n in [(0, 50), (17, 40), (300, 5)]:
        pos = np.arange(hist, hist + n)
        assert visible_pairs(hist, n, kind, window) == int(visible_mask(pos, hist + n, kind, window).sum())


def test_pages_figures(golden_dir):
    with open(os.path.join(golden_dir, "pages_figures.json")) as f:
        fig = json.load(f)
    assert fig["layers_swa"] + fig["layers_full"] == fig["layers_total"]
    assert fig["layers_swa"] == fig["swa_per_full"] * fig["layers_full"]
    W = fig["window"]
    # The 1/7 figures are the long-sequence limit of the hybrid/all-full ratios.
    for n in (1 << 16, 1 << 20):
        kv = hybrid_kv_ratio(n, fig["layers_swa"], fig["layers_full"], W)
        assert kv == pytest.approx(fig["kv_ratio_approx"], abs=0.002)
    pairs = hybrid_prefill_pair_ratio(1 << 20, fig["layers_swa"], fig["layers_full"], W)
    assert pairs == pytest.approx(fig["prefill_compute_ratio_approx"], abs=0.001)
    # Short sequences (N <= W) get no saving at all.
    assert hybrid_kv_ratio(W, fig["layers_swa"], fig["layers_full"], W) == 1.0


def test_kv_rows_is_window_bounded():
    assert kv_rows(10, "swa", 128) == 10
    assert kv_rows(10**6, "swa", 128) == 128
    assert kv_rows(10**6, "full", 128) == 10**6
    assert visible_keys(0, "swa", 128) == 1
    assert visible_keys(500, "swa", 128) == 128
