"""Hand-worked prefix-cache cases (tests/golden/prefix_cache_cases.json),
replayed on the brute-force model in oracle/prefix_cache.py alone, then on
the library's tree. Each case names the reading it follows: which ring a
position's SWA KV comes from, how pages are owned, and how rings leave the
cache (youleyou.com "小米MiMo首次公开模型推理系统全链路优化降价99%", section 2
"KVCache系统重构：让缓存真正省下来"). Host-only: no GPU."""

import json
import os

import numpy as np
import pytest

from oracle.prefix_cache import PrefixCacheModel
from oracle.window_safe import window_safe_length


def _load(golden_dir):
    with open(os.path.join(golden_dir, "prefix_cache_cases.json")) as f:
        data = json.load(f)
    assert data["source"] and data["cases"]
    return data


# What each kind of operation is expected to return (the other fields are its arguments).
_EXPECTED = {
    "insert": ("kept", "ring_kept"),
    "match": ("matched", "valid", "ring", "pages", "reuse"),
    "advance": (),
    "release": (),
    "evict_swa": ("freed",),
}


def _replay(data, case, apply):
    """Runs one case's operations through `apply(op)`, which returns the
    observed results as a dict (or raises for a refused call)."""
    for i, op in enumerate(case["ops"]):
        what = f"{case['name']} [{case['reading']}], op {i} ({op['op']}): {op.get('why', '')}"
        if op.get("error"):
            with pytest.raises((ValueError, RuntimeError)):
                apply(op)
            continue
        got = apply(op)
        for key in _EXPECTED[op["op"]]:
            assert got[key] == op[key], f"{what}: {key} = {got[key]}, expected {op[key]}"


def test_model_reproduces_the_hand_worked_cases(golden_dir):
    data = _load(golden_dir)
    w, ps = data["window"], data["page_size"]
    for case in data["cases"]:
        model = PrefixCacheModel(w, ps)

        def apply(op):
            kind = op["op"]
            if kind == "insert":
                kept, ring_kept = model.insert(op["tokens"], op["pages"], op["ring"], op["ring_len"], op["transfer"])
                return {"kept": kept, "ring_kept": ring_kept}
            if kind == "match":
                m, valid, ring, pages = model.match(op["tokens"])
                reuse = window_safe_length(op["tokens"], op["tokens"][:m], valid[:m], w)
                assert max(model.positions_per_ring().values(), default=0) <= w
                return {"matched": m, "valid": valid, "ring": ring, "pages": pages, "reuse": reuse}
            if kind == "advance":
                model.ring_advance(op["ring"], op["len"])
                return {}
            if kind == "release":
                model.ring_release(op["ring"])
                return {}
            if kind == "evict_swa":
                return {"freed": model.evict_swa(op["want"])}
            raise AssertionError(kind)

        _replay(data, case, apply)


def test_library_tree_reproduces_the_hand_worked_cases(golden_dir):
    from hybrid_sliding_window_gqa_amd import window_safe_match
    from hybrid_sliding_window_gqa_amd._lib import HybridAttnError
    from hybrid_sliding_window_gqa_amd.prefix_tree import PrefixTree

    data = _load(golden_dir)
    w, ps = data["window"], data["page_size"]
    for case in data["cases"]:
        tree = PrefixTree(w, ps)

        def apply(op):
            kind = op["op"]
            try:
                if kind == "insert":
                    kept, ring_kept = tree.insert(op["tokens"], op["pages"], op["ring"], op["ring_len"],
                                                  op["transfer"])
                    return {"kept": kept.tolist(), "ring_kept": ring_kept}
                if kind == "match":
                    r = tree.match(op["tokens"])
                    toks = np.asarray(op["tokens"], np.int32)
                    reuse = window_safe_match(toks, toks[:r.matched], r.swa_valid[:r.matched], w)
                    assert tree.stats()["most_positions_per_ring"] <= w
                    return {"matched": r.matched, "valid": r.swa_valid.tolist(), "ring": r.swa_ring.tolist(),
                            "pages": r.pages.tolist(), "reuse": reuse}
                if kind == "advance":
                    tree.ring_advance(op["ring"], op["len"])
                    return {}
                if kind == "release":
                    tree.ring_release(op["ring"])
                    return {}
                if kind == "evict_swa":
                    return {"freed": tree.evict_swa(op["want"]).tolist()}
            except HybridAttnError as e:
                raise RuntimeError(str(e)) from e
            raise AssertionError(kind)

        _replay(data, case, apply)
        tree.close()
