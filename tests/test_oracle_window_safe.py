"""Pins for oracle.window_safe: hand-worked cases from the pages' rule and
structural properties over exhaustive tiny inputs."""

import itertools
import json
import os

import pytest

from oracle.window_safe import common_prefix_length, window_safe_length


def _case_inputs(case):
    n = case["cached_len"]
    cached = list(range(100, 100 + n))
    lcp = case["lcp"]
    request = cached[:lcp] + [-1] * 3          # diverges right after the common prefix
    valid = [1] * n
    for p in case["evicted"]:
        valid[p] = 0
    return request, cached, valid


def test_golden_cases(golden_dir):
    with open(os.path.join(golden_dir, "window_safe_cases.json")) as f:
        data = json.load(f)
    assert data["source"]
    for case in data["cases"]:
        request, cached, valid = _case_inputs(case)
        got = window_safe_length(request, cached, valid, case["window"])
        assert got == case["expect"], case["name"]


def test_common_prefix_length():
    assert common_prefix_length([1, 2, 3], [1, 2, 4]) == 2
    assert common_prefix_length([1, 2], [1, 2, 3]) == 2
    assert common_prefix_length([], [1]) == 0


@pytest.mark.parametrize("window", [1, 2, 3, 5])
def test_exhaustive_properties(window):
    n = 9
    cached = list(range(n))
    for bits in itertools.product([0, 1], repeat=n):
        for m in range(n + 1):
            request = cached[:m] + [-7]
            L = window_safe_length(request, cached, bits, window)
            assert 0 <= L <= m
            # The chosen length is safe ...
            assert all(bits[j] for j in range(max(0, L - window), L))
            # ... and clipping happens only when it must: all valid => no clipping.
            if all(bits[:m]):
                assert L == m
            # Making one more slot valid never shrinks the reusable length.
            for j in range(n):
                if not bits[j]:
                    more = list(bits)
                    more[j] = 1
                    assert window_safe_length(request, cached, more, window) >= L
            # Evictions older than the last window of the match never matter.
            if m >= window:
                cleared = [1] * (m - window) + list(bits[m - window:])
                assert window_safe_length(request, cached, cleared, window) == L or not all(
                    bits[m - window : m]
                )


def test_rejects_bad_arguments():
    with pytest.raises(ValueError):
        window_safe_length([1], [1], [1], 0)
    with pytest.raises(ValueError):
        window_safe_length([1], [1, 2], [1], 4)
