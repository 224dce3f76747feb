"""The library's window_safe_match (C++, host) against the oracle's brute force:
exhaustively on tiny inputs, randomly up to the reuse workload's sizes, and on
the hand-worked golden cases. Bit-exact (an integer length)."""

import itertools
import json
import os

import numpy as np
import pytest

import synth
from hybrid_sliding_window_gqa_amd import HybridAttnError, window_safe_match
from oracle.window_safe import window_safe_length


@pytest.mark.parametrize("window", [1, 2, 3, 4, 5])
def test_exhaustive_tiny(window):
    n = 8
    cached = np.arange(n, dtype=np.int32)
    for bits in itertools.product([0, 1], repeat=n):
        valid = np.array(bits, dtype=np.uint8)
        for m in range(n + 1):
            req = np.concatenate([cached[:m], np.array([-5], np.int32)])
            assert window_safe_match(req, cached, valid, window) == window_safe_length(req, cached, valid, window)


def test_random_long():
    rng = np.random.default_rng(11)
    for trial in range(60):
        n = int(rng.integers(1, 4096))
        window = int(rng.choice([1, 7, 16, 128, 300]))
        cached = rng.integers(0, 5, size=n).astype(np.int32)
        m = int(rng.integers(0, n + 1))
        req = np.concatenate([cached[:m], rng.integers(5, 9, size=int(rng.integers(0, 5))).astype(np.int32)])
        valid = (rng.random(n) > rng.choice([0.0, 0.001, 0.02, 0.3])).astype(np.uint8)
        assert window_safe_match(req, cached, valid, window) == window_safe_length(req, cached, valid, window)


def test_golden_cases(golden_dir):
    with open(os.path.join(golden_dir, "window_safe_cases.json")) as f:
        cases = json.load(f)["cases"]
    for case in cases:
        n = case["cached_len"]
        cached = np.arange(100, 100 + n, dtype=np.int32)
        req = np.concatenate([cached[: case["lcp"]], np.array([-1, -1], np.int32)])
        valid = np.ones(n, np.uint8)
        valid[case["evicted"]] = 0
        assert window_safe_match(req, cached, valid, case["window"]) == case["expect"], case["name"]


def test_reuse_workload_lengths():
    s = synth.reuse_structure()
    for b in range(s.batch):
        req, cached, valid = synth.reuse_tokens(s, b)
        got = window_safe_match(req, cached, valid, 128)
        assert got == window_safe_length(req, cached, valid, 128)
        ev = s.extra["evicted"][b]
        assert got == (int(ev.min()) if len(ev) else int(s.hist[b]))


def test_rejects_bad_input():
    with pytest.raises(HybridAttnError):
        window_safe_match([1], [1], [1], 0)
    with pytest.raises(ValueError):
        window_safe_match([1], [1, 2], [1], 4)
