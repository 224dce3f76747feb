"""Oracle: a brute-force prefix cache for the dual-pool KV cache (test
infrastructure only: nothing on the product path imports it).

What a prefix cache must answer under sliding-window layers
(youleyou.com "小米MiMo首次公开模型推理系统全链路优化降价99%", section 2
"KVCache系统重构：让缓存真正省下来"; blog.hotdry.top 2026-06-09, section
"Hybrid SWA：用 1/7 计算量捕获长程依赖"): equal token prefixes no longer mean
the KV is all there. Each cached position keeps a Full page (long-lived) and,
separately, an SWA source that disappears when the ring holding it moves on or
is freed -- the tree's nodes carry both maps and evict them independently,
SWA eviction follows the request's lifecycle, and the match handed to the
window-safe rule carries the SWA validity of every matched position.

This model keeps no tree at all. A cached position is identified by its token
prefix (the tuple of tokens up to and including it), so "the cached paths" are
the set of such tuples, and every question is answered by looking tuples up:
    page_of[prefix]  -> Full page id recorded for that position's page index
    src[prefix]      -> id of the ring holding that position's SWA KV
    rings[id]        -> owned flag, last use, the prefixes it holds
The pages fix what the cache must answer (a match whose SWA map feeds the
window-safe rule; Full and SWA parts evicted independently; SWA eviction tied
to the request's lifecycle, so a ring never names more than W positions) but
not who owns which KV or in which order rings leave. The rules below are the
plainest readings that fit, each pinned by hand-worked cases in
tests/golden/prefix_cache_cases.json (reading ids as given there):
  - R19, SWA sources: a request's ring holds its last W positions. A position
    has one source: a position without one takes the inserting ring; a
    position held by a live ring moves to a ring that is handed over (the
    live one will move on, the handed-over one stays); otherwise the first
    source stays. A ring that already held positions keeps only its window
    at ring_len.
  - R20, pages: paths are token-granular; a cached position keeps its page,
    a new position takes the caller's page for its page index. The match
    reports, for page index i, the page of position min(m, (i + 1) * ps) - 1.
  - R21, lifecycle: a live ring drops positions below new_len - W when its
    request advances and all of them on release; handed-over rings leave only
    by SWA eviction, least recently used first, ties by lower ring id. The
    clock ticks once per insert and per match; an insert marks its ring used,
    a match marks every ring it reports.
Full eviction (whole least-recently-used leaves) depends on where a tree's
nodes are split and is not modelled: tests check its invariants and re-sync
this model from the tree's answers with forget().
"""

from __future__ import annotations


class PrefixCacheModel:
    def __init__(self, window: int, page_size: int):
        self.w, self.ps = int(window), int(page_size)
        self.page_of = {}      # prefix tuple -> page id
        self.src = {}          # prefix tuple -> ring id
        self.rings = {}        # ring id -> {"owned": bool, "use": int, "held": set of prefix tuples}
        self.clock = 0

    # -- helpers ---------------------------------------------------------------
    def matched(self, tokens) -> int:
        m = 0
        while m < len(tokens) and tuple(tokens[: m + 1]) in self.page_of:
            m += 1
        return m

    def _drop_below(self, rid: int, lo: int) -> None:
        ring = self.rings[rid]
        for key in [k for k in ring["held"] if len(k) - 1 < lo]:
            ring["held"].discard(key)
            del self.src[key]

    # -- operations ------------------------------------------------------------
    def insert(self, tokens, pages, ring_id=-1, ring_len=0, transfer=False):
        tokens = [int(t) for t in tokens]
        n = len(tokens)
        if ring_id >= 0 and ring_id in self.rings and self.rings[ring_id]["owned"]:
            raise ValueError("ring belongs to the tree")   # refused: nothing changes
        self.clock += 1
        for q in range(n):
            key = tuple(tokens[: q + 1])
            if key not in self.page_of:
                self.page_of[key] = int(pages[q // self.ps])
        ring_kept = False
        if ring_id >= 0:
            ring = self.rings.setdefault(ring_id, {"owned": False, "use": 0, "held": set()})
            ring["owned"] = bool(transfer)
            ring["use"] = self.clock
            self._drop_below(ring_id, ring_len - self.w)
            for p in range(max(0, ring_len - self.w), min(ring_len, n)):
                key = tuple(tokens[: p + 1])
                old = self.src.get(key)
                if old == ring_id:
                    continue
                if old is not None:
                    if self.rings[old]["owned"] or not ring["owned"]:
                        continue
                    self.rings[old]["held"].discard(key)
                self.src[key] = ring_id
                ring["held"].add(key)
            ring_kept = bool(ring["held"])
            if not ring_kept:
                del self.rings[ring_id]
        referenced = set(self.page_of.values())
        kept = [1 if int(p) in referenced else 0 for p in pages]
        return kept, ring_kept

    def match(self, tokens):
        tokens = [int(t) for t in tokens]
        n = len(tokens)
        self.clock += 1
        m = self.matched(tokens)
        valid, ring = [0] * n, [-1] * n
        for p in range(m):
            rid = self.src.get(tuple(tokens[: p + 1]))
            if rid is not None:
                valid[p], ring[p] = 1, rid
                self.rings[rid]["use"] = self.clock
        pages = []
        for i in range(-(-n // self.ps)):
            if i * self.ps >= m:
                pages.append(-1)
            else:
                last = min(m, (i + 1) * self.ps) - 1
                pages.append(self.page_of[tuple(tokens[: last + 1])])
        return m, valid, ring, pages

    def ring_advance(self, rid: int, new_len: int) -> None:
        if rid not in self.rings:
            return
        if self.rings[rid]["owned"]:
            raise ValueError("ring belongs to the tree")
        self._drop_below(rid, new_len - self.w)
        if not self.rings[rid]["held"]:
            del self.rings[rid]

    def ring_release(self, rid: int) -> None:
        if rid not in self.rings:
            return
        if self.rings[rid]["owned"]:
            raise ValueError("ring belongs to the tree")
        self._drop_below(rid, 1 << 62)
        del self.rings[rid]

    def evict_swa(self, want: int):
        order = sorted((r["use"], rid) for rid, r in self.rings.items() if r["owned"])
        freed = [rid for _, rid in order[:want]]
        for rid in freed:
            self._drop_below(rid, 1 << 62)
            del self.rings[rid]
        return freed

    def forget(self, prefixes) -> None:
        """Remove cached positions (after a Full eviction in the tree)."""
        for key in prefixes:
            self.page_of.pop(key, None)
            rid = self.src.pop(key, None)
            if rid is not None:
                ring = self.rings[rid]
                ring["held"].discard(key)
                if not ring["held"]:
                    del self.rings[rid]

    def positions_per_ring(self) -> dict:
        return {rid: len(r["held"]) for rid, r in self.rings.items()}
