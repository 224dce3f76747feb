"""Mutation checks of the oracle's pins (CPU only).

A pin is only worth something if a plausible slip in the oracle fails it.
Each mutant below is a copy of an oracle function with one planted mistake;
the test runs the existing pins against it and requires at least one of them
to fail. The oracle itself is never modified: the mutants live here."""

import math

import numpy as np
import pytest

import test_oracle_attention as pins
import test_prefix_cache_golden as golden
from oracle.prefix_cache import PrefixCacheModel
from oracle.window_safe import window_safe_length


# ---- attention: the masked-softmax definition with one mistake each ---------

def _mutant_attend(mistake):
    def attend(q, k, v, q_pos, kind, window, scale=None):
        q = np.asarray(q, dtype=np.float64)
        n, hq, d = q.shape
        hkv = k.shape[1]
        if hq % hkv != 0 or kind not in ("swa", "full"):
            raise ValueError("bad arguments")
        q_pos = np.asarray(q_pos, dtype=np.int64)
        if n and (q_pos.min() < 0 or q_pos.max() >= k.shape[0]):
            raise ValueError("query position outside the key range")
        if scale is None:
            scale = 1.0 / math.sqrt(d)
        if mistake == "no_scale":
            scale = 1.0
        last = int(q_pos.max()) + 1 if n else 0
        t = q_pos[:, None]
        j = np.arange(last)[None, :]
        mask = (j >= t) if mistake == "anti_causal" else (j <= t)
        if kind == "swa":
            lo = t - window if mistake == "window_plus_one" else t - window + 1
            mask = mask & (j >= lo)
        out = np.zeros((n, hq, d))
        lse = np.zeros((n, hq))
        group = hq // hkv
        for h in range(hq):
            g = h % hkv if mistake == "gqa_interleaved" else h // group
            kg = np.asarray(k[:last, g], np.float64)
            vg = np.asarray(v[:last, g], np.float64)
            if mistake == "transposed_v":
                vg = vg[::-1]
            s = np.where(mask, scale * (q[:, h] @ kg.T), -np.inf)
            m = s.max(axis=1, keepdims=True)
            if mistake == "lse_log2":
                l = m[:, 0] + np.log2(np.exp(s - m).sum(axis=1))
            else:
                l = m[:, 0] + np.log(np.exp(s - m).sum(axis=1))
            p = np.exp(s - (m if mistake == "unnormalised" else l[:, None]))
            out[:, h] = p @ vg
            lse[:, h] = l
        return out, lse
    return attend


ATTENTION_PINS = [
    lambda: pins.test_all_equal_keys_closed_form("swa", 3),
    lambda: pins.test_all_equal_keys_closed_form("full", 4),
    pins.test_window_one_is_self_only,
    lambda: pins.test_swa_equals_full_when_window_covers_sequence(16),
    pins.test_window_changes_result_when_shorter,
    lambda: pins.test_matches_torch_sdpa("swa", 5, 8, 2),
    lambda: pins.test_matches_torch_sdpa("full", 0, 4, 1),
    pins.test_gqa_equals_mha_with_repeated_kv,
    lambda: pins.test_scalar_bruteforce_tiny("swa", 3),
    pins.test_single_row_equals_row_of_full_prefill,
]


def _failures(pin_list):
    failed = 0
    for pin in pin_list:
        try:
            pin()
        except AssertionError:
            failed += 1
    return failed


def test_unmutated_copy_passes_every_pin(monkeypatch):
    monkeypatch.setattr(pins, "attend", _mutant_attend(None))
    assert _failures(ATTENTION_PINS) == 0


@pytest.mark.parametrize("mistake", ["no_scale", "anti_causal", "window_plus_one", "gqa_interleaved",
                                     "transposed_v", "lse_log2", "unnormalised"])
def test_attention_mistake_fails_a_pin(monkeypatch, mistake):
    monkeypatch.setattr(pins, "attend", _mutant_attend(mistake))
    assert _failures(ATTENTION_PINS) >= 1, mistake


# ---- window-safe rule --------------------------------------------------------

def _ws_mutant(mistake):
    def ws(request, cached, valid, window):
        m = 0
        while m < min(len(request), len(cached)) and request[m] == cached[m]:
            m += 1
        w = window - 1 if mistake == "w_minus_one" else window
        for length in range(m, -1, -1):
            lo = max(0, length - w)
            hi = length + 1 if mistake == "includes_next" else length
            if all(valid[j] for j in range(lo, min(hi, len(valid)))):
                return length
        return 0
    return ws


@pytest.mark.parametrize("mistake", ["w_minus_one", "includes_next"])
def test_window_safe_mistake_fails_a_golden_case(golden_dir, mistake):
    import json
    import os

    import test_oracle_window_safe as ws_pins
    with open(os.path.join(golden_dir, "window_safe_cases.json")) as f:
        cases = json.load(f)["cases"]
    fn = _ws_mutant(mistake)
    wrong = 0
    for case in cases:
        request, cached, valid = ws_pins._case_inputs(case)
        wrong += fn(request, cached, valid, case["window"]) != case["expect"]
    assert wrong >= 1
    for case in cases:                              # and the real rule gets every case right
        request, cached, valid = ws_pins._case_inputs(case)
        assert window_safe_length(request, cached, valid, case["window"]) == case["expect"]


# ---- prefix cache model ------------------------------------------------------

class _EvictMostRecent(PrefixCacheModel):
    def evict_swa(self, want):
        order = sorted(((r["use"], rid) for rid, r in self.rings.items() if r["owned"]), reverse=True)
        freed = [rid for _, rid in order[:want]]
        for rid in freed:
            self._drop_below(rid, 1 << 62)
            del self.rings[rid]
        return freed


class _TiesByHigherId(PrefixCacheModel):
    def evict_swa(self, want):
        order = sorted((r["use"], -rid) for rid, r in self.rings.items() if r["owned"])
        freed = [-nrid for _, nrid in order[:want]]
        for rid in freed:
            self._drop_below(rid, 1 << 62)
            del self.rings[rid]
        return freed


class _MatchMarksNothing(PrefixCacheModel):
    def match(self, tokens):
        uses = {rid: r["use"] for rid, r in self.rings.items()}
        res = super().match(tokens)
        for rid, u in uses.items():
            if rid in self.rings:
                self.rings[rid]["use"] = u
        return res


class _AdvanceKeepsOneMore(PrefixCacheModel):
    def ring_advance(self, rid, new_len):
        super().ring_advance(rid, new_len - 1)


class _RingHoldsWPlusOne(PrefixCacheModel):
    def __init__(self, window, page_size):
        super().__init__(window, page_size)

    def insert(self, tokens, pages, ring_id=-1, ring_len=0, transfer=False):
        self.w += 1
        try:
            return super().insert(tokens, pages, ring_id, ring_len, transfer)
        finally:
            self.w -= 1


class _NewestSourceWins(PrefixCacheModel):
    """Any inserting ring takes every position in its window."""

    def insert(self, tokens, pages, ring_id=-1, ring_len=0, transfer=False):
        if ring_id >= 0:
            for p in range(max(0, ring_len - self.w), min(ring_len, len(tokens))):
                key = tuple(int(t) for t in tokens[: p + 1])
                old = self.src.pop(key, None)
                if old is not None:
                    self.rings[old]["held"].discard(key)
        return super().insert(tokens, pages, ring_id, ring_len, transfer)


class _PageOfFirstPosition(PrefixCacheModel):
    def match(self, tokens):
        m, valid, ring, pages = super().match(tokens)
        tokens = [int(t) for t in tokens]
        pages = [self.page_of[tuple(tokens[: i * self.ps + 1])] if i * self.ps < m else -1
                 for i in range(len(pages))]
        return m, valid, ring, pages


class _CallerPageWins(PrefixCacheModel):
    def insert(self, tokens, pages, ring_id=-1, ring_len=0, transfer=False):
        for q in range(len(tokens)):
            self.page_of.pop(tuple(int(t) for t in tokens[: q + 1]), None)
        return super().insert(tokens, pages, ring_id, ring_len, transfer)


MODEL_MUTANTS = [_EvictMostRecent, _TiesByHigherId, _MatchMarksNothing, _AdvanceKeepsOneMore,
                 _RingHoldsWPlusOne, _NewestSourceWins, _PageOfFirstPosition, _CallerPageWins]


def _golden_failures(golden_dir, model_cls):
    data = golden._load(golden_dir)
    w, ps = data["window"], data["page_size"]
    failed = 0
    for case in data["cases"]:
        model = model_cls(w, ps)

        def apply(op):
            kind = op["op"]
            if kind == "insert":
                kept, ring_kept = model.insert(op["tokens"], op["pages"], op["ring"], op["ring_len"], op["transfer"])
                return {"kept": kept, "ring_kept": ring_kept}
            if kind == "match":
                m, valid, ring, pages = model.match(op["tokens"])
                reuse = window_safe_length(op["tokens"], op["tokens"][:m], valid[:m], w)
                return {"matched": m, "valid": valid, "ring": ring, "pages": pages, "reuse": reuse}
            if kind == "advance":
                model.ring_advance(op["ring"], op["len"])
                return {}
            if kind == "release":
                model.ring_release(op["ring"])
                return {}
            return {"freed": model.evict_swa(op["want"])}

        try:
            golden._replay(data, case, apply)
        except (AssertionError, pytest.fail.Exception, KeyError, ValueError):
            failed += 1
    return failed


def test_real_model_passes_the_golden_cases(golden_dir):
    assert _golden_failures(golden_dir, PrefixCacheModel) == 0


@pytest.mark.parametrize("mutant", MODEL_MUTANTS, ids=lambda c: c.__name__.lstrip("_"))
def test_prefix_model_mistake_fails_a_golden_case(golden_dir, mutant):
    assert _golden_failures(golden_dir, mutant) >= 1
