"""Pins for oracle.indexing: ring slots against a deque model and a closed form,
page locations against a permutation's coverage."""

import collections

import numpy as np
import pytest

from oracle.indexing import page_location, pages_needed, ring_contents, ring_slot


@pytest.mark.parametrize("window", [1, 3, 4, 16, 128])
@pytest.mark.parametrize("start,count", [(0, 0), (0, 1), (0, 5), (0, 300), (37, 200), (1000, 3)])
def test_ring_equals_last_w_appended(window, start, count):
    appended = list(range(start, start + count))
    slots = ring_contents(appended, window)
    # deque(maxlen=W) keeps exactly the last W appended positions.
    last_w = list(collections.deque(appended, maxlen=window))
    held = sorted(int(p) for p in slots if p >= 0)
    assert held == last_w
    for s, p in enumerate(slots):
        if p >= 0:
            assert p % window == s


@pytest.mark.parametrize("window", [4, 128])
def test_ring_closed_form(window):
    n = 3 * window + 5
    slots = ring_contents(range(n), window)
    for s in range(window):
        expect = s + window * ((n - 1 - s) // window) if s < n else -1
        assert slots[s] == expect


def test_ring_restore_from_prefix_window():
    # Restoring a cached prefix of reusable length L into a fresh ring writes
    # positions L-W .. L-1; the ring then holds exactly those.
    W, L = 8, 29
    slots = ring_contents(range(L - W, L), W)
    assert sorted(slots.tolist()) == list(range(L - W, L))
    assert ring_slot(L - 1, W) == (L - 1) % W


def test_ring_rejects_unordered():
    with pytest.raises(ValueError):
        ring_contents([3, 2], 4)


def test_page_location_covers_each_slot_once():
    rng = np.random.default_rng(0)
    page_size, tokens = 16, 16 * 9 + 5
    n_pages = pages_needed(tokens, page_size)
    assert n_pages == 10
    table = rng.permutation(40)[:n_pages]
    pages, offs = page_location(table, np.arange(tokens), page_size)
    pairs = set(zip(pages.tolist(), offs.tolist()))
    assert len(pairs) == tokens
    assert set(pages.tolist()) == set(table.tolist())
    assert offs.max() == page_size - 1
    # consecutive positions stay within one page until a page boundary
    assert all(pages[p] == pages[p - 1] for p in range(1, tokens) if p % page_size)


def test_page_location_rejects_overflow():
    with pytest.raises(ValueError):
        page_location([3, 4], 32, 16)
