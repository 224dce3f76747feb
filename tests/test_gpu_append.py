"""a1 / a2 on the GPU: appended K/V land exactly where the oracle's ring and
page models say, bit-exact, and nothing else in the pools changes."""

import numpy as np
import pytest
import torch

import hybrid_sliding_window_gqa_amd as ha
from gpu_util import DEV, append_history, check_pages, check_ring, host, i32, make_generator, page_blocks, randn_bf16
from oracle.indexing import page_location

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("window,hkv,d", [(32, 2, 64), (128, 8, 128), (16, 1, 64)])
@pytest.mark.parametrize("src", [torch.bfloat16, torch.float32])
def test_ring_append_sequence_of_calls(window, hkv, d, src):
    shape = ha.HeadShape(hkv * 2, hkv, d, window=window)
    gen = make_generator(101)
    lens = [1, window - 1, window + 5, 3 * window + 7]
    total = max(lens) + 40
    seq = [(randn_bf16(gen, total, hkv, d), randn_bf16(gen, total, hkv, d)) for _ in lens]
    if src == torch.float32:
        # float32 sources: the library rounds to bf16 (nearest-even); feed
        # float32 copies that differ from the bf16 values below the bf16 ulp.
        noise = [(k.float() + 1e-4 * torch.randn(k.shape, generator=gen, device="cuda"),
                  v.float() - 1e-4 * torch.randn(v.shape, generator=gen, device="cuda")) for k, v in seq]
        expect = [(a.to(torch.bfloat16), b.to(torch.bfloat16)) for a, b in noise]
        feed = noise
    else:
        expect = feed = seq
    pool = ha.SwaRingPool(shape, num_rings=len(lens) + 3, device="cuda", fill=float("nan"))
    ring_id = [4, 0, 6, 2]
    view = pool.view(i32(ring_id))
    # Append in three calls with different chunk sizes per sequence.
    cuts = [[0, 0, 1], [0, 3, window - 1], [0, window, window + 5], [0, 17, 2 * window + 1]]
    for step in range(3):
        starts = [c[step] for c in cuts]
        ends = [cuts[b][step + 1] if step + 1 < 3 else lens[b] for b in range(len(lens))]
        append_history(shape, view, feed, starts, ends)
    torch.cuda.synchronize()
    for b, n in enumerate(lens):
        k_h = host(expect[b][0])
        v_h = host(expect[b][1])
        check_ring(pool, ring_id[b], k_h, v_h, list(range(n)), window)
    # rings no sequence owns stay untouched
    for r in set(range(pool.num_rings)) - set(ring_id):
        assert torch.isnan(pool.k[r].float()).all() and torch.isnan(pool.v[r].float()).all()


@pytest.mark.parametrize("window,hkv,d", [(1, 2, 64), (3, 1, 64), (24, 2, 128), (100, 8, 64)])
def test_ring_append_windows_not_a_multiple_of_16(window, hkv, d):
    # the ring is ceil(W / 16) blocks; slot p mod W, padding slots never written
    shape = ha.HeadShape(hkv * 2, hkv, d, window=window)
    gen = make_generator(303 + window)
    lens = [1, window + 2, 3 * window + 5, 50]
    seq = [(randn_bf16(gen, n, hkv, d), randn_bf16(gen, n, hkv, d)) for n in lens]
    pool = ha.SwaRingPool(shape, num_rings=len(lens) + 2, device="cuda", fill=float("nan"))
    ring_id = [3, 0, 5, 1]
    view = pool.view(i32(ring_id))
    cuts = [sorted({0, min(n, 2), min(n, window + 1), n}) for n in lens]
    for step in range(max(len(c) for c in cuts) - 1):
        starts = [c[min(step, len(c) - 1)] for c in cuts]
        ends = [c[min(step + 1, len(c) - 1)] for c in cuts]
        append_history(shape, view, seq, starts, ends)
    torch.cuda.synchronize()
    for b, n in enumerate(lens):
        check_ring(pool, ring_id[b], host(seq[b][0]), host(seq[b][1]), list(range(n)), window)
    for r in set(range(pool.num_rings)) - set(ring_id):
        assert torch.isnan(pool.k[r].float()).all() and torch.isnan(pool.v[r].float()).all()


@pytest.mark.parametrize("page_size", [16, 64])
@pytest.mark.parametrize("hkv,d", [(1, 64), (8, 128)])
def test_page_append_permuted_table(hkv, d, page_size):
    # a page of 64 tokens holds four 16-token blocks per kv head
    shape = ha.HeadShape(hkv * 4, hkv, d, page_size=page_size)
    gen = make_generator(202)
    rng = np.random.default_rng(5)
    lens = [5, 16, 33, 300]
    pages_per = [-(-n // page_size) for n in lens]
    num_pages = sum(pages_per) + 9
    perm = rng.permutation(num_pages)
    stride = max(pages_per) + 2
    table = np.full((len(lens), stride), -1, np.int32)
    off = 0
    for b, c in enumerate(pages_per):
        table[b, :c] = perm[off:off + c]
        off += c
    seq = [(randn_bf16(gen, n, hkv, d), randn_bf16(gen, n, hkv, d)) for n in lens]
    pool = ha.FullPagePool(shape, num_pages, device="cuda", fill=float("nan"))
    view = pool.view(i32(table))
    # two calls: a prefix, then the rest (positions continue mid-page)
    mid = [n // 3 for n in lens]
    append_history(shape, view, seq, [0] * len(lens), mid)
    append_history(shape, view, seq, mid, lens)
    torch.cuda.synchronize()
    used = set()
    for b, n in enumerate(lens):
        check_pages(pool, table[b], host(seq[b][0]), host(seq[b][1]), n)
        used |= set(table[b, :pages_per[b]].tolist())
        # tail of the last page is untouched
        last = table[b, pages_per[b] - 1]
        tail = n - page_size * (pages_per[b] - 1)
        for g in range(hkv):
            kb, vb = page_blocks(pool, g)
            assert np.isnan(kb[last, tail:]).all() and np.isnan(vb[last, tail:]).all()
    for p in set(range(num_pages)) - used:
        assert torch.isnan(pool.k[p].float()).all() and torch.isnan(pool.v[p].float()).all()


def test_out_of_range_ids_are_dropped():
    shape = ha.HeadShape(4, 1, 64)
    gen = make_generator(303)
    pool = ha.FullPagePool(shape, 4, device="cuda", fill=float("nan"))
    table = np.array([[2, 99, -1, 1]], np.int32)   # 99 and -1 are not pages of this pool
    seq = [(randn_bf16(gen, 64, 1, 64), randn_bf16(gen, 64, 1, 64))]
    append_history(shape, pool.view(i32(table)), seq, [0], [64])
    ring = ha.SwaRingPool(shape, 2, device="cuda", fill=float("nan"))
    append_history(shape, ring.view(i32([7])), seq, [0], [20])
    torch.cuda.synchronize()
    k = host(seq[0][0])
    kb, _ = page_blocks(pool, 0)
    np.testing.assert_array_equal(kb[2], k[0:16, 0])
    np.testing.assert_array_equal(kb[1], k[48:64, 0])
    assert torch.isnan(pool.k[0].float()).all() and torch.isnan(pool.k[3].float()).all()
    assert torch.isnan(ring.k.float()).all()


@pytest.mark.parametrize("page_size", [16, 32])
@pytest.mark.parametrize("src", [torch.bfloat16, torch.float32])
@pytest.mark.parametrize("hkv,d", [(2, 64), (8, 128)])
def test_page_block_append_matches_row_append(src, hkv, d, page_size):
    """A full-pool call that brings at least 16 tokens per sequence on average
    is written page block by page block; the same call with the batch padded
    by empty sequences takes the per-row path. Both must write the same
    slots with the same bits (untouched slots keep their NaN), and those
    slots must be where the oracle's page model puts each position.
    Starts are unaligned, page-aligned and negative (positions below 0 are
    dropped); float32 sources are rounded to bfloat16 on the way. Pages of
    32 tokens hold two 16-token blocks per kv head."""
    shape = ha.HeadShape(hkv * 4, hkv, d, page_size=page_size)
    gen = make_generator(404 + d + hkv)
    rng = np.random.default_rng(9)
    starts = [0, 5, 16, 37, -3]
    counts = [40, 11, 64, 100, 30]
    ends = [s + c for s, c in zip(starts, counts)]
    pages_per = [-(-max(e, 0) // page_size) for e in ends]
    num_pages = sum(pages_per) + 5
    perm = rng.permutation(num_pages)
    stride = max(pages_per) + 1
    table = np.full((len(starts), stride), -1, np.int32)
    off = 0
    for b, c in enumerate(pages_per):
        table[b, :c] = perm[off:off + c]
        off += c
    total = sum(counts)
    k_new = torch.randn(total, hkv, d, generator=gen, device=DEV)
    v_new = torch.randn(total, hkv, d, generator=gen, device=DEV)
    if src == torch.bfloat16:
        k_new, v_new = k_new.to(torch.bfloat16), v_new.to(torch.bfloat16)
    expect_k, expect_v = host(k_new.to(torch.bfloat16)), host(v_new.to(torch.bfloat16))
    cu = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    pad = 4 * len(starts)                      # average falls below 16 tokens per sequence
    pools = []
    for extra in (0, pad):
        pool = ha.FullPagePool(shape, num_pages, device=DEV, fill=float("nan"))
        tab = np.concatenate([table, np.full((extra, stride), -1, np.int32)])
        pos0 = np.concatenate([starts, np.zeros(extra, np.int32)])
        cu_b = np.concatenate([cu, np.full(extra, total, np.int32)])
        ha.full_pool_append(shape, pool.view(i32(tab)), i32(pos0), i32(cu_b), k_new.contiguous(), v_new.contiguous())
        pools.append(pool)
    torch.cuda.synchronize()
    a, b_ = pools
    assert torch.equal(a.k.view(torch.int16), b_.k.view(torch.int16))
    assert torch.equal(a.v.view(torch.int16), b_.v.view(torch.int16))
    written = np.zeros((num_pages, page_size), bool)
    for g in range(hkv):
        kb, vb = page_blocks(a, g)
        for b in range(len(starts)):
            pos = np.arange(max(starts[b], 0), ends[b])
            pages, offs = page_location(table[b], pos, page_size)
            rows = cu[b] + (pos - starts[b])
            np.testing.assert_array_equal(kb[pages, offs], expect_k[rows, g])
            np.testing.assert_array_equal(vb[pages, offs], expect_v[rows, g])
            written[pages, offs] = True
        assert np.isnan(kb[~written]).all() and np.isnan(vb[~written]).all()
