"""a1 / a2 on the GPU: appended K/V land exactly where the oracle's ring and
page models say, bit-exact, and nothing else in the pools changes."""

import numpy as np
import pytest
import torch

import hybrid_sliding_window_gqa_amd as ha
from gpu_util import append_history, check_pages, check_ring, host, i32, make_generator, page_blocks, randn_bf16

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


@pytest.mark.parametrize("hkv,d", [(1, 64), (8, 128)])
def test_page_append_permuted_table(hkv, d):
    shape = ha.HeadShape(hkv * 4, hkv, d)
    gen = make_generator(202)
    rng = np.random.default_rng(5)
    lens = [5, 16, 33, 300]
    pages_per = [-(-n // 16) for n in lens]
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
        tail = n - 16 * (pages_per[b] - 1)
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
