"""The benchmark's algorithmic work counts -- the numerators of every GB/s,
TFLOP/s and roofline fraction it prints -- against brute-force counts over
the oracle's visibility mask (oracle/attention.py visible_mask), for small
shapes, windows 1, 3, 24 and 128, and both layer kinds."""

import numpy as np
import pytest

import bench
import hybrid_sliding_window_gqa_amd as ha
from oracle.attention import visible_mask

KINDS = ("swa", "full")
WINDOWS = (1, 3, 24, 128)


def shape(window):
    return ha.HeadShape(8, 2, 64, window=window)


def seen(q_pos, num_keys, kind, window):
    """Number of (query, key) pairs the mask admits, and the set of key
    positions any of the queries sees."""
    m = visible_mask(np.asarray(q_pos), num_keys, kind, window)
    return int(m.sum()), set(np.nonzero(m.any(axis=0))[0].tolist())


@pytest.mark.parametrize("kind", KINDS)
@pytest.mark.parametrize("window", WINDOWS)
def test_visible_pairs_range_counts_the_mask(kind, window):
    for hist, n in ((0, 1), (0, 37), (5, 200), (130, 64), (1000, 17)):
        want, _ = seen(np.arange(hist, hist + n), hist + n, kind, window)
        assert bench.visible_pairs_range(hist, n, kind, window) == want


@pytest.mark.parametrize("kind", KINDS)
@pytest.mark.parametrize("window", WINDOWS)
def test_decode_bytes_count_the_keys_the_query_sees(kind, window):
    s = shape(window)
    kv_len = np.array([1, 2, 16, 17, 129, 300])
    tok = s.num_kv_heads * s.head_dim * 2 * 2
    keys = sum(seen([n - 1], n, kind, window)[0] for n in kv_len)
    qol = len(kv_len) * s.num_q_heads * (s.head_dim * 2 + s.head_dim * 4 + 4)
    assert bench.decode_layer_bytes(s, kind, kv_len) == keys * tok + qol


@pytest.mark.parametrize("kind", KINDS)
@pytest.mark.parametrize("window", WINDOWS)
@pytest.mark.parametrize("kv8", [False, True])
def test_verify_bytes_count_history_keys_once(kind, window, kv8):
    # history keys any of the nq queries sees are read once; the new tokens
    # are read as bf16 and written in the pool's format
    s = shape(window)
    nq = 4
    t0 = np.array([0, 1, 5, 40, 129, 300])
    tok = s.num_kv_heads * s.head_dim * 2 * 2
    pool_tok = s.num_kv_heads * (s.head_dim * 2 + 8) if kv8 else tok
    hist_keys = 0
    for t in t0:
        _, keys = seen(np.arange(t, t + nq), t + nq, kind, window)
        hist_keys += sum(1 for j in keys if j < t)
    qol = len(t0) * nq * s.num_q_heads * (s.head_dim * 2 + s.head_dim * 4 + 4)
    want = hist_keys * pool_tok + len(t0) * nq * (tok + pool_tok) + qol
    assert bench.verify_layer_bytes(s, kind, t0, nq, kv8) == want


def test_int8_token_bytes():
    s = shape(128)
    assert bench.kv8_bytes_per_token(s) == s.num_kv_heads * (s.head_dim + s.head_dim + 4 + 4)


@pytest.mark.parametrize("window", WINDOWS)
def test_prefill_pass_flops_count_the_mask(window):
    s = shape(window)
    kinds = ["swa"] * 6 + ["full"]
    batch, total, chunk = 2, 96, 32
    got = bench.prefill_pass_flops(s, kinds, batch, total, chunk)
    for kind in KINDS:
        pairs, _ = seen(np.arange(total), total, kind, window)      # chunking does not change the pairs
        want = pairs * batch * s.num_q_heads * 4 * s.head_dim * kinds.count(kind)
        assert got[kind] == want
