"""The library's prefix tree (include/prefix_tree.h) against the brute-force
model in oracle/prefix_cache.py and against what the pages state: reuse is
cut to the window-safe length, a ring that moved on or was freed makes a
token-equal prefix a "false hit" that must not be reused, SWA occupancy
stays at W positions per ring, and Full and SWA segments are evicted
independently (youleyou.com "小米MiMo首次公开模型推理系统全链路优化降价99%",
section 2 "KVCache系统重构：让缓存真正省下来"). Host-only: no GPU."""

import numpy as np
import pytest

from hybrid_sliding_window_gqa_amd import _lib
from hybrid_sliding_window_gqa_amd.prefix_tree import PrefixTree
from oracle.prefix_cache import PrefixCacheModel
from oracle.window_safe import window_safe_length

W, PS = 8, 4


def pages_for(n, start=100):
    return list(range(start, start + -(-n // PS)))


def test_multi_turn_extension_reuses_everything_with_one_copied_page():
    tree = PrefixTree(W, PS)
    a = list(range(1, 23))                         # 22 tokens: page index 5 holds 20, 21
    kept, ring_kept = tree.insert(a, pages_for(22), ring_id=0, ring_len=22, transfer=True)
    assert kept.tolist() == [1] * 6 and ring_kept
    b = a + [50, 51, 52, 53, 54]
    r = tree.reuse(b)
    assert (r.matched, r.length) == (22, 22)
    assert r.shared_pages.tolist() == pages_for(22)[:5]
    assert r.cow_page == pages_for(22)[5]          # positions 20, 21 are copied, not written in place
    assert r.window_rings.tolist() == [0] * W
    st = tree.stats()
    assert (st["owned_rings"], st["swa_positions"], st["most_positions_per_ring"]) == (1, W, W)


def test_false_hit_after_the_owner_ring_moved_on():
    tree = PrefixTree(W, PS)
    a = list(range(1, 23))
    tree.insert(a, pages_for(22), ring_id=1, ring_len=22)      # live request
    tree.ring_advance(1, 25)                                     # it decoded 3 more tokens
    b = a + [60, 61]
    m = tree.match(b)
    assert m.matched == 22                                       # token-equal prefix ...
    assert m.swa_valid[:22].tolist() == [0] * 17 + [1] * 5      # ... but only [17, 22) still in the ring
    r = tree.reuse(b)
    assert r.length == 0                                         # no window of W valid positions
    assert window_safe_length(b, b[:22], m.swa_valid[:22], W) == 0


def test_release_and_independent_eviction():
    tree = PrefixTree(W, PS)
    a = list(range(1, 23))
    tree.insert(a, pages_for(22), ring_id=2, ring_len=22)
    tree.ring_release(2)                                         # request ended without handing over
    m = tree.match(a)
    assert m.matched == 22 and not m.swa_valid.any()
    assert tree.reuse(a).length == 0
    # a finished request hands its ring over; SWA eviction frees only the ring
    b = [9] + a
    tree.insert(b, pages_for(23, 200), ring_id=3, ring_len=23, transfer=True)
    assert tree.reuse(b).length == 23
    assert tree.evict_swa(5).tolist() == [3]
    m = tree.match(b)
    assert m.matched == 23 and not m.swa_valid.any()
    assert m.pages.tolist() == pages_for(23, 200)               # Full segment intact
    freed, rings = tree.evict_full(1 << 20)
    assert sorted(freed.tolist()) == sorted(pages_for(22) + pages_for(23, 200)) and rings.size == 0
    assert tree.stats()["nodes"] == 0 and tree.stats()["pages"] == 0


def test_lru_leaf_eviction_and_locks():
    tree = PrefixTree(W, PS)
    seqs = [[k] + list(range(10, 17)) for k in (1, 2, 3)]        # three disjoint 8-token paths, 2 pages each
    for i, s in enumerate(seqs):
        tree.insert(s, pages_for(8, 10 * i))
    tree.match(seqs[0])                                          # most recent: 0; oldest: 1
    freed, _ = tree.evict_full(1)
    assert sorted(freed.tolist()) == pages_for(8, 10)
    tree.lock(seqs[2], 5)                                        # splits path 2 at position 5
    freed, _ = tree.evict_full(1 << 20)
    # path 0 goes; of path 2 only the unlocked tail [5, 8) goes, and it shares page index 1 with the head
    assert sorted(freed.tolist()) == pages_for(8, 0)
    assert tree.match(seqs[2]).matched == 5
    tree.unlock(seqs[2], 5)
    freed, _ = tree.evict_full(1 << 20)
    assert sorted(freed.tolist()) == pages_for(8, 20)
    with pytest.raises(_lib.HybridAttnError):
        tree.unlock(seqs[2], 5)


def test_split_pages_are_freed_once():
    tree = PrefixTree(W, PS)
    a = list(range(1, 23))
    tree.insert(a, pages_for(22, 100))
    b = a[:10] + [70, 71, 72, 73, 74, 75]                        # diverges inside page index 2
    own = pages_for(16, 300)
    kept, _ = tree.insert(b, [100, 101] + own[2:])
    assert kept.tolist() == [1, 1, 1, 1]                         # pages 100, 101 are the tree's; 302, 303 new
    m = tree.match(b)
    assert m.pages.tolist() == [100, 101, 302, 303]
    assert tree.match(a).pages.tolist() == pages_for(22, 100)
    freed = []
    while True:
        f, _ = tree.evict_full(1)
        if f.size == 0 and tree.stats()["nodes"] == 0:
            break
        freed += f.tolist()
    assert sorted(freed) == sorted(pages_for(22, 100) + [302, 303])


def test_new_positions_must_not_reuse_a_tree_page():
    tree = PrefixTree(W, PS)
    a = list(range(1, 23))
    tree.insert(a, pages_for(22))
    b = a[:10] + [80, 81]                                        # position 10 lands in the tree's page 102
    with pytest.raises(_lib.HybridAttnError) as e:
        tree.insert(b, pages_for(12))
    assert e.value.status == _lib.HA_ERR_RANGE
    assert tree.match(b).matched == 10                           # nothing changed


def test_argument_errors():
    tree = PrefixTree(W, PS)
    with pytest.raises(ValueError):
        tree.insert([1, 2, 3], [1, 2])
    with pytest.raises(_lib.HybridAttnError):
        tree.insert([1, 2, 3], [-1])
    tree.insert([1, 2, 3], [5], ring_id=4, ring_len=3, transfer=True)
    for call in (lambda: tree.ring_advance(4, 9), lambda: tree.ring_release(4),
                 lambda: tree.insert([1, 2, 3], [5], ring_id=4, ring_len=3)):
        with pytest.raises(_lib.HybridAttnError):
            call()
    with pytest.raises(_lib.HybridAttnError):
        tree.lock([1, 2, 3, 4], 4)                               # only 3 positions cached
    tree.ring_advance(77, 5)                                     # unknown live rings are ignored
    tree.ring_release(77)


def test_model_on_the_pages_scenarios():
    """The model alone: a handed-over ring makes a multi-turn extension fully
    reusable; a live ring that moved on leaves a token-equal prefix that the
    window-safe rule refuses; a ring never names more than W positions."""
    a = list(range(1, 23))
    model = PrefixCacheModel(W, PS)
    model.insert(a, pages_for(22), ring_id=0, ring_len=22, transfer=True)
    m, valid, ring, pages = model.match(a + [50])
    assert m == 22 and valid[:22] == [0] * 14 + [1] * 8 and pages == pages_for(22)
    assert window_safe_length(a + [50], a, valid[:22], W) == 22
    model = PrefixCacheModel(W, PS)
    model.insert(a, pages_for(22), ring_id=1, ring_len=22)
    model.ring_advance(1, 25)
    m, valid, _, _ = model.match(a)
    assert m == 22 and window_safe_length(a, a, valid, W) == 0
    assert max(model.positions_per_ring().values()) == 5 <= W


class Driver:
    """Random requests over a tiny vocabulary (so paths share prefixes), run
    on the tree and on the model side by side."""

    def __init__(self, seed):
        self.rng = np.random.default_rng(seed)
        self.tree, self.model = PrefixTree(W, PS), PrefixCacheModel(W, PS)
        self.live = {}            # ring id -> tokens of its request (length = ring length)
        self.known = []           # every token list inserted
        self.locks = []
        self.next_ring = 0
        self.next_page = 1000
        self.free_pages = []

    def fresh_page(self):
        if self.free_pages and self.rng.random() < 0.5:
            return self.free_pages.pop(int(self.rng.integers(len(self.free_pages))))
        self.next_page += 1
        return self.next_page

    def tokens(self, n):
        return [int(x) for x in self.rng.integers(0, 3, n)]

    def base(self):
        if self.known and self.rng.random() < 0.8:
            s = self.known[int(self.rng.integers(len(self.known)))]
            return list(s[: int(self.rng.integers(0, len(s) + 1))])
        return []

    def insert(self, toks, ring_id=-1, ring_len=0, transfer=False):
        m = self.model.matched(toks)
        pages = []
        for i in range(-(-len(toks) // PS)):
            if (i + 1) * PS <= m and self.rng.random() < 0.5:
                pages.append(self.model.page_of[tuple(toks[: (i + 1) * PS])])   # borrowed
            else:
                pages.append(self.fresh_page())
        kept, ring_kept = self.tree.insert(toks, pages, ring_id, ring_len, transfer)
        mk, mrk = self.model.insert(toks, pages, ring_id, ring_len, transfer)
        assert kept.tolist() == mk and ring_kept == mrk
        for p, k in zip(pages, kept):
            if not k and p not in self.model.page_of.values():
                self.free_pages.append(p)
        self.known.append(list(toks))

    def check_match(self, toks):
        got = self.tree.match(toks)
        m, valid, ring, pages = self.model.match(toks)
        assert got.matched == m
        assert got.swa_valid.tolist() == valid and got.swa_ring.tolist() == ring
        assert got.pages.tolist() == pages
        # the window-safe length the tree's map yields equals brute force over the model's map
        assert self.tree.reuse(toks).length == window_safe_length(toks, toks[:m], valid[:m], W)
        self.model.match(toks)                         # reuse() matched once more

    def check_stats(self):
        st = self.tree.stats()
        per_ring = {r: c for r, c in self.model.positions_per_ring().items() if c}
        assert st["pages"] == len(set(self.model.page_of.values()))
        assert st["swa_positions"] == len(self.model.src) == sum(per_ring.values())
        assert st["owned_rings"] == sum(1 for r in self.model.rings.values() if r["owned"])
        assert st["most_positions_per_ring"] == max(per_ring.values(), default=0) <= W

    def evict_full(self, want):
        owned_before = {r for r, v in self.model.rings.items() if v["owned"]}
        pages_before = set(self.model.page_of.values())
        freed, rings = self.tree.evict_full(want)
        lost = []
        for s in self.known:
            m_tree = self.tree.match(s).matched
            lost += [tuple(s[: q + 1]) for q in range(m_tree, self.model.matched(s))]
        self.model.forget(set(lost))
        for s in self.known:                           # the same matches on the model, in the same order
            self.model.match(s)
        pages_after = set(self.model.page_of.values())
        assert sorted(freed.tolist()) == sorted(pages_before - pages_after)
        owned_after = {r for r, v in self.model.rings.items() if v["owned"]}
        assert sorted(rings.tolist()) == sorted(owned_before - owned_after)
        for toks, n in self.locks:
            assert self.model.matched(toks) >= n
        self.free_pages += freed.tolist()

    def step(self):
        op = self.rng.random()
        if op < 0.2 or not self.live:                              # a new request
            rid = self.next_ring
            self.next_ring += 1
            toks = self.base() + self.tokens(int(self.rng.integers(1, 20)))
            self.live[rid] = toks
            if self.rng.random() < 0.5:
                self.insert(toks, rid, len(toks))
        elif op < 0.35:                                            # decode steps of a live request
            rid = list(self.live)[int(self.rng.integers(len(self.live)))]
            self.live[rid] += self.tokens(int(self.rng.integers(1, 6)))
            self.tree.ring_advance(rid, len(self.live[rid]))
            self.model.ring_advance(rid, len(self.live[rid]))
        elif op < 0.45:                                            # insert a live request (maybe a prefix)
            rid = list(self.live)[int(self.rng.integers(len(self.live)))]
            toks = self.live[rid]
            n = len(toks) if self.rng.random() < 0.6 else int(self.rng.integers(0, len(toks) + 1))
            self.insert(toks[:n], rid, len(toks))
        elif op < 0.6:                                             # a request ends
            rid = list(self.live)[int(self.rng.integers(len(self.live)))]
            toks = self.live.pop(rid)
            if self.rng.random() < 0.75:
                self.insert(toks, rid, len(toks), transfer=True)
            else:
                self.tree.ring_release(rid)
                self.model.ring_release(rid)
        elif op < 0.8:
            self.check_match(self.base() + self.tokens(int(self.rng.integers(0, 6))))
        elif op < 0.85:
            want = int(self.rng.integers(1, 3))
            assert self.tree.evict_swa(want).tolist() == self.model.evict_swa(want)
        elif op < 0.9 and self.known:
            s = self.known[int(self.rng.integers(len(self.known)))]
            n = min(self.model.matched(s), int(self.rng.integers(0, len(s) + 1)))
            self.tree.lock(s, n)
            self.locks.append((s, n))
        elif op < 0.93 and self.locks:
            s, n = self.locks.pop(int(self.rng.integers(len(self.locks))))
            self.tree.unlock(s, n)
        elif op < 0.96:
            self.evict_full(int(self.rng.integers(1, 6)))
        self.check_stats()


@pytest.mark.parametrize("seed", range(12))
def test_random_operations_match_the_model(seed):
    d = Driver(seed)
    for _ in range(400):
        d.step()
    for s in d.known[-20:]:
        d.check_match(s + [0])
