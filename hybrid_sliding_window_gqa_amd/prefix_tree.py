"""Host prefix cache over the dual-pool KV cache (include/prefix_tree.h).

A radix tree in the library whose nodes carry a Full page index and an SWA
segment map; its match emits the validity map window_safe_match consumes
(youleyou.com "小米MiMo首次公开模型推理系统全链路优化降价99%", section 2
"KVCache系统重构：让缓存真正省下来": window-safe matching, SWA eviction tied
to the request's lifecycle, Full and SWA segments evicted independently).
This module only marshals arrays; every step runs in the library.
"""

from __future__ import annotations

import ctypes
from dataclasses import dataclass

import numpy as np

from ._lib import check, load
from .api import window_safe_match


@dataclass
class Match:
    matched: int              # longest cached prefix m
    swa_valid: np.ndarray     # uint8 [n]: position p < m held by a ring
    swa_ring: np.ndarray      # int32 [n]: that ring, -1 if none
    pages: np.ndarray         # int32 [ceil(n / page_size)]: page ids along the path, -1 past m


@dataclass
class Reuse:
    """What a request may reuse: positions [0, length) of its prefix."""

    length: int               # window-safe length L (<= matched)
    matched: int              # longest cached prefix m
    shared_pages: np.ndarray  # page ids of page indices [0, L // page_size): reference as they are
    cow_page: int             # page id to copy for index L // page_size when L is not page-aligned, else -1
    window_rings: np.ndarray  # int32 [min(L, W)]: ring holding each of positions [L - min(L, W), L)


def _i32(x) -> np.ndarray:
    return np.ascontiguousarray(x, dtype=np.int32)


class PrefixTree:
    """One tree per model (pages and rings are shared by its layers)."""

    def __init__(self, window: int = 128, page_size: int = 16):
        self._lib = load()
        self.window, self.page_size = int(window), int(page_size)
        handle = ctypes.c_void_p()
        check(self._lib.ha_tree_create(self.window, self.page_size, ctypes.byref(handle)))
        self._h = handle

    def close(self) -> None:
        if self._h:
            self._lib.ha_tree_destroy(self._h)
            self._h = ctypes.c_void_p()

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def _np(self, n: int) -> int:
        return -(-n // self.page_size)

    def insert(self, tokens, pages, ring_id: int = -1, ring_len: int = 0, transfer: bool = False):
        """Cache a request's tokens; returns (page_kept uint8 [ceil(n/ps)], ring_kept bool)."""
        tok, pg = _i32(tokens), _i32(pages)
        if pg.size != self._np(tok.size):
            raise ValueError(f"{tok.size} tokens need {self._np(tok.size)} page ids, got {pg.size}")
        kept = np.zeros(pg.size, np.uint8)
        ring_kept = ctypes.c_int32(0)
        check(self._lib.ha_tree_insert(self._h, tok.ctypes.data, tok.size, pg.ctypes.data, int(ring_id),
                                       int(ring_len), int(bool(transfer)), kept.ctypes.data,
                                       ctypes.byref(ring_kept)))
        return kept, bool(ring_kept.value)

    def match(self, tokens) -> Match:
        tok = _i32(tokens)
        n = tok.size
        valid = np.zeros(n, np.uint8)
        ring = np.full(n, -1, np.int32)
        pages = np.full(self._np(n), -1, np.int32)
        m = ctypes.c_int64(0)
        check(self._lib.ha_tree_match(self._h, tok.ctypes.data, n, ctypes.byref(m), valid.ctypes.data,
                                      ring.ctypes.data, pages.ctypes.data))
        return Match(int(m.value), valid, ring, pages)

    def reuse(self, tokens) -> Reuse:
        """Match, then cut to the window-safe length with the library's window_safe_match."""
        tok = _i32(tokens)
        mt = self.match(tok)
        m, w, ps = mt.matched, self.window, self.page_size
        length = window_safe_match(tok, tok[:m], mt.swa_valid[:m], w)
        shared = mt.pages[: length // ps].copy()
        cow = int(mt.pages[length // ps]) if length % ps else -1
        if length % ps and cow < 0:
            raise RuntimeError("no page for the partly reused page index")
        return Reuse(length, m, shared, cow, mt.swa_ring[length - min(length, w):length].copy())

    def lock(self, tokens, n: int) -> None:
        tok = _i32(tokens)
        check(self._lib.ha_tree_lock(self._h, tok.ctypes.data, int(n), 1))

    def unlock(self, tokens, n: int) -> None:
        tok = _i32(tokens)
        check(self._lib.ha_tree_lock(self._h, tok.ctypes.data, int(n), -1))

    def ring_advance(self, ring_id: int, new_len: int) -> None:
        check(self._lib.ha_tree_ring_advance(self._h, int(ring_id), int(new_len)))

    def ring_release(self, ring_id: int) -> None:
        check(self._lib.ha_tree_ring_release(self._h, int(ring_id)))

    def evict_full(self, want_pages: int, page_cap: int | None = None, ring_cap: int = 1 << 16):
        """Returns (freed page ids, freed tree-owned ring ids)."""
        page_cap = max(int(want_pages), 1) * 4 + 4096 if page_cap is None else int(page_cap)
        pages = np.zeros(max(page_cap, 1), np.int32)
        rings = np.zeros(max(ring_cap, 1), np.int32)
        n_p, n_r = ctypes.c_int64(0), ctypes.c_int64(0)
        check(self._lib.ha_tree_evict_full(self._h, int(want_pages), pages.ctypes.data, page_cap, ctypes.byref(n_p),
                                           rings.ctypes.data, ring_cap, ctypes.byref(n_r)))
        return pages[: n_p.value].copy(), rings[: n_r.value].copy()

    def evict_swa(self, want_rings: int) -> np.ndarray:
        cap = max(int(want_rings), 1)
        rings = np.zeros(cap, np.int32)
        n_r = ctypes.c_int64(0)
        check(self._lib.ha_tree_evict_swa(self._h, int(want_rings), rings.ctypes.data, cap, ctypes.byref(n_r)))
        return rings[: n_r.value].copy()

    def stats(self) -> dict:
        out = np.zeros(6, np.int64)
        check(self._lib.ha_tree_stats(self._h, out.ctypes.data))
        keys = ("nodes", "pages", "swa_positions", "owned_rings", "live_rings", "most_positions_per_ring")
        return dict(zip(keys, (int(x) for x in out)))
