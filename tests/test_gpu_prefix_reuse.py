"""Window-safe prefix reuse end to end on the GPU: the library's prefix tree
decides what a new request may reuse; its window moves from the source ring
into the new request's ring and the partly shared page is copied, both with
the pool read and append calls; the new tokens' prefill over those pools
then matches the oracle (max |O| error <= 1e-2, max |LSE| error <= 1e-3) and
leaves the cached request's pages untouched (youleyou.com
"小米MiMo首次公开模型推理系统全链路优化降价99%", section 2
"KVCache系统重构：让缓存真正省下来")."""

import numpy as np
import pytest
import torch

import hybrid_sliding_window_gqa_amd as ha
from gpu_util import assert_close, host, i32, make_generator, oracle_rows, randn_bf16
from hybrid_sliding_window_gqa_amd.prefix_tree import PrefixTree

pytestmark = pytest.mark.gpu

W = 32


def test_read_returns_what_was_appended():
    shape = ha.HeadShape(8, 2, 128, window=W)
    lens = [5, 40, 100]
    gen = make_generator(1)
    k = [randn_bf16(gen, n, 2, 128) for n in lens]
    v = [randn_bf16(gen, n, 2, 128) for n in lens]
    ring = ha.SwaRingPool(shape, 3, "cuda", fill=float("nan"))
    pages = ha.FullPagePool(shape, 16, "cuda", fill=float("nan"))
    perm = np.random.default_rng(0).permutation(16)
    table = np.full((3, 7), -1, np.int32)
    table[0, :1], table[1, :3], table[2, :7] = perm[:1], perm[1:4], perm[4:11]
    rv, pv = ring.view(i32([2, 0, 1])), pages.view(i32(table))
    cu = i32(np.concatenate([[0], np.cumsum(lens)]))
    kc, vc = torch.cat(k).contiguous(), torch.cat(v).contiguous()
    ha.swa_ring_append(shape, rv, i32([0, 0, 0]), cu, kc, vc)
    ha.full_pool_append(shape, pv, i32([0, 0, 0]), cu, kc, vc)
    # pages: every position; ring: the last min(n, W) positions
    ko, vo = torch.empty_like(kc), torch.empty_like(vc)
    ha.full_pool_read(shape, pv, i32([0, 0, 0]), cu, ko, vo)
    torch.cuda.synchronize()
    assert torch.equal(ko.view(torch.int16), kc.view(torch.int16)) and torch.equal(vo.view(torch.int16),
                                                                                   vc.view(torch.int16))
    first = [max(0, n - W) for n in lens]
    cnt = [n - f for n, f in zip(lens, first)]
    rk = torch.empty(sum(cnt), 2, 128, dtype=torch.bfloat16, device="cuda")
    rvv = torch.empty_like(rk)
    ha.swa_ring_read(shape, rv, i32(first), i32(np.concatenate([[0], np.cumsum(cnt)])), rk, rvv)
    torch.cuda.synchronize()
    want_k = torch.cat([x[f:] for x, f in zip(k, first)])
    want_v = torch.cat([x[f:] for x, f in zip(v, first)])
    assert torch.equal(rk.view(torch.int16), want_k.view(torch.int16))
    assert torch.equal(rvv.view(torch.int16), want_v.view(torch.int16))


@pytest.mark.parametrize("page_size", [16, 64])
@pytest.mark.parametrize("cached,new", [(300, 40), (256, 17), (45, 80)])
def test_tree_driven_reuse_matches_the_oracle(cached, new, page_size):
    ps = page_size
    shape = ha.HeadShape(16, 2, 128, window=W, page_size=ps)
    total = cached + new
    gen = make_generator(cached + new)
    rng = np.random.default_rng(cached)
    tok_a = rng.integers(0, 50000, cached).tolist()
    tok_b = tok_a + rng.integers(0, 50000, new).tolist()
    kinds = (ha.HA_SWA, ha.HA_FULL)
    kv = {kd: (randn_bf16(gen, total, 2, 128), randn_bf16(gen, total, 2, 128), randn_bf16(gen, total, 16, 128))
          for kd in kinds}                                   # B's logical K, V, Q; A's are the first `cached`
    npg = 64
    alloc = ha.PageAllocator(npg, np.random.default_rng(5).permutation(npg))
    rings = ha.SwaRingPool(shape, 4, "cuda", fill=float("nan"))
    pools = ha.FullPagePool(shape, npg, "cuda", fill=float("nan"))
    # request A: its K/V in ring 0 and its pages, then handed to the tree
    pages_a = alloc.alloc(-(-cached // ps))
    ring_a, table_a = rings.view(i32([0])), pools.view(i32([pages_a]))
    one = lambda n: i32([0, n])
    ha.swa_ring_append(shape, ring_a, i32([0]), one(cached), kv[ha.HA_SWA][0][:cached].contiguous(),
                       kv[ha.HA_SWA][1][:cached].contiguous())
    ha.full_pool_append(shape, table_a, i32([0]), one(cached), kv[ha.HA_FULL][0][:cached].contiguous(),
                        kv[ha.HA_FULL][1][:cached].contiguous())
    tree = PrefixTree(W, ps)
    kept, ring_kept = tree.insert(tok_a, pages_a, ring_id=0, ring_len=cached, transfer=True)
    assert kept.all() and ring_kept
    snapshot = pools.k.clone(), pools.v.clone()
    # request B: what the tree lets it reuse
    r = tree.reuse(tok_b)
    assert r.matched == cached and r.length == cached        # the whole cached request, window-safe
    assert r.shared_pages.tolist() == pages_a[: cached // ps]
    assert set(r.window_rings.tolist()) == {0}
    tree.lock(tok_b, r.length)
    n_pages_b = -(-total // ps)
    own = alloc.alloc(n_pages_b - len(r.shared_pages))
    pages_b = r.shared_pages.tolist() + own
    ring_b, table_b = rings.view(i32([1])), pools.view(i32([pages_b]))
    L = r.length
    if r.cow_page >= 0:                                      # copy the partly shared page before writing to it
        p0 = (L // ps) * ps
        ko = torch.empty(L - p0, 2, 128, dtype=torch.bfloat16, device="cuda")
        vo = torch.empty_like(ko)
        ha.full_pool_read(shape, table_a, i32([p0]), one(L - p0), ko, vo)
        ha.full_pool_append(shape, table_b, i32([p0]), one(L - p0), ko, vo)
    w0 = L - min(L, W)                                       # the window, from the ring the tree names
    ko = torch.empty(L - w0, 2, 128, dtype=torch.bfloat16, device="cuda")
    vo = torch.empty_like(ko)
    ha.swa_ring_read(shape, rings.view(i32([int(r.window_rings[0])])), i32([w0]), one(L - w0), ko, vo)
    ha.swa_ring_append(shape, ring_b, i32([w0]), one(L - w0), ko, vo)
    # prefill B's new tokens over the reused pools
    for kd, view in ((ha.HA_SWA, ring_b), (ha.HA_FULL, table_b)):
        k, v, q = kv[kd]
        out, lse = ha.hybrid_attn_prefill(shape, view, i32([L]), one(total - L), q[L:].contiguous(),
                                          k[L:].contiguous(), v[L:].contiguous(), max_new=total - L)
        torch.cuda.synchronize()
        rows = np.arange(L, total)
        ref_o, ref_l = oracle_rows(host(q)[rows], host(k), host(v), rows, "swa" if kd == ha.HA_SWA else "full", W)
        assert_close(host(out), host(lse), ref_o, ref_l, f"kind {kd}")
        fn = ha.swa_ring_append if kd == ha.HA_SWA else ha.full_pool_append
        fn(shape, view, i32([L]), one(total - L), k[L:].contiguous(), v[L:].contiguous())
    torch.cuda.synchronize()
    # A's pages were never written by B
    for a_pg in pages_a:
        assert torch.equal(pools.k[a_pg].view(torch.int16), snapshot[0][a_pg].view(torch.int16))
        assert torch.equal(pools.v[a_pg].view(torch.int16), snapshot[1][a_pg].view(torch.int16))
    # B finishes: the tree keeps the shared pages, takes B's own pages and ring
    tree.unlock(tok_b, L)
    kept, ring_kept = tree.insert(tok_b, pages_b, ring_id=1, ring_len=total, transfer=True)
    assert kept.all() and ring_kept
    assert tree.reuse(tok_b + [7]).length == total
