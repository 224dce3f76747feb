"""Physical placement never changes a result (reading R13: page placement and
ring ids are the caller's choice; the Full pool's page table is the
authoritative index -- youleyou.com "小米MiMo首次公开模型推理系统全链路优化降价99%",
section 2 "KVCache系统重构：让缓存真正省下来"). Prefill, multi-token verify and
INT8-pool decode give bit-identical outputs for two different page
permutations and two different ring-id assignments of the same logical K/V."""

import numpy as np
import pytest
import torch

import hybrid_sliding_window_gqa_amd as ha
from gpu_util import DEV, append_history, cu_from_counts, i32, make_generator, randn_bf16

pytestmark = pytest.mark.gpu

SHAPE = ha.HeadShape(64, 8, 128)


def logical(lens, seed):
    gen = make_generator(seed)
    hkv, d = SHAPE.num_kv_heads, SHAPE.head_dim
    return [(randn_bf16(gen, n, hkv, d), randn_bf16(gen, n, hkv, d)) for n in lens]


def full_view(lens, perm_seed, kv_dtype="bf16"):
    per = [-(-n // 16) for n in lens]
    num_pages = sum(per) + 7
    perm = np.random.default_rng(perm_seed).permutation(num_pages)
    table = np.full((len(lens), max(per) + 1), -1, np.int32)
    off = 0
    for b, c in enumerate(per):
        table[b, :c] = perm[off:off + c]
        off += c
    pool = ha.FullPagePool(SHAPE, num_pages, DEV, fill=float("nan"), kv_dtype=kv_dtype)
    return pool, pool.view(i32(table))


def ring_view(ring_ids, kv_dtype="bf16"):
    pool = ha.SwaRingPool(SHAPE, max(ring_ids) + 1, DEV, fill=float("nan"), kv_dtype=kv_dtype)
    return pool, pool.view(i32(ring_ids))


PLACEMENTS = {
    ha.HA_FULL: [dict(perm_seed=1), dict(perm_seed=2)],
    ha.HA_SWA: [dict(ring_ids=[0, 1, 2]), dict(ring_ids=[5, 2, 0])],
}


def make_view(kind, placement, kv_dtype="bf16"):
    if kind == ha.HA_FULL:
        return full_view(placement["lens"], placement["perm_seed"], kv_dtype)
    return ring_view(placement["ring_ids"], kv_dtype)


@pytest.mark.parametrize("kind", [ha.HA_SWA, ha.HA_FULL])
def test_prefill_is_placement_invariant(kind):
    hist, new = [300, 0, 1501], [40, 129, 64]
    totals = [h + n for h, n in zip(hist, new)]
    seq = logical(totals, seed=21)
    gen = make_generator(22)
    q = randn_bf16(gen, sum(new), SHAPE.num_q_heads, SHAPE.head_dim)
    cat = lambda i: torch.cat([s[i][h:t] for s, h, t in zip(seq, hist, totals)]).contiguous()
    results = []
    for placement in PLACEMENTS[kind]:
        pool, view = make_view(kind, dict(placement, lens=totals))
        append_history(SHAPE, view, seq, [0] * 3, hist)
        out, lse = ha.hybrid_attn_prefill(SHAPE, view, i32(hist), i32(cu_from_counts(new)), q, cat(0), cat(1),
                                          max_new=max(new))
        torch.cuda.synchronize()
        results.append((out, lse))
    assert torch.equal(results[0][0], results[1][0]) and torch.equal(results[0][1], results[1][1])


@pytest.mark.parametrize("kind", [ha.HA_SWA, ha.HA_FULL])
@pytest.mark.parametrize("kv_dtype", ["bf16", "int8"])
def test_verify_is_placement_invariant(kind, kv_dtype):
    nq = 4
    lens = [25, 700, 2049]
    seq = logical(lens, seed=31)
    gen = make_generator(32)
    q = randn_bf16(gen, len(lens), nq, SHAPE.num_q_heads, SHAPE.head_dim)
    rows = lambda i: torch.stack([s[i][n - nq:n] for s, n in zip(seq, lens)]).contiguous()
    results = []
    for placement in PLACEMENTS[kind]:
        pool, view = make_view(kind, dict(placement, lens=lens), kv_dtype)
        append_history(SHAPE, view, seq, [0] * 3, [n - nq for n in lens])
        out, lse = ha.hybrid_attn_verify(SHAPE, view, i32(lens), q, rows(0), rows(1), max(lens), num_splits=3)
        torch.cuda.synchronize()
        results.append((out, lse))
    assert torch.equal(results[0][0], results[1][0]) and torch.equal(results[0][1], results[1][1])


@pytest.mark.parametrize("kind", [ha.HA_SWA, ha.HA_FULL])
@pytest.mark.parametrize("fused", [False, True])
def test_int8_decode_is_placement_invariant(kind, fused):
    lens = [17, 129, 3000]
    seq = logical(lens, seed=41)
    gen = make_generator(42)
    q = randn_bf16(gen, len(lens), SHAPE.num_q_heads, SHAPE.head_dim)
    results = []
    for placement in PLACEMENTS[kind]:
        pool, view = make_view(kind, dict(placement, lens=lens), kv_dtype="int8")
        hist = [n - 1 for n in lens] if fused else lens
        append_history(SHAPE, view, seq, [0] * 3, hist)
        kw = {}
        if fused:
            kw = dict(k_new=torch.stack([s[0][n - 1] for s, n in zip(seq, lens)]).contiguous(),
                      v_new=torch.stack([s[1][n - 1] for s, n in zip(seq, lens)]).contiguous())
        out, lse = ha.hybrid_attn_decode(SHAPE, view, i32(lens), q, max(lens), num_splits=4, **kw)
        torch.cuda.synchronize()
        results.append((out, lse))
    assert torch.equal(results[0][0], results[1][0]) and torch.equal(results[0][1], results[1][1])
