"""a6 / a7 / a8 on the GPU: decode over ring and page pools matches the oracle
(max |O| error <= 1e-2, max |LSE| error <= 1e-3), for ragged lengths that
span window edges, page edges, split-K and empty rows; results are
bit-invariant to physical page order and ring id."""

import numpy as np
import pytest
import torch

import hybrid_sliding_window_gqa_amd as ha
from gpu_util import (
    append_history,
    assert_close,
    host,
    i32,
    make_generator,
    oracle_rows,
    randn_bf16,
)

pytestmark = pytest.mark.gpu

LENS = [1, 2, 15, 16, 17, 127, 128, 129, 130, 300, 1000, 2049]


def build(shape, kind, lens, seed, table_perm_seed=0, ring_order=None, appended=None):
    """Pools holding each sequence's positions [0, appended[b]) (default: all
    lens[b]), page tables sized for lens[b] tokens."""
    gen = make_generator(seed)
    hkv, d = shape.num_kv_heads, shape.head_dim
    seq = [(randn_bf16(gen, max(n, 1), hkv, d), randn_bf16(gen, max(n, 1), hkv, d)) for n in lens]
    q = randn_bf16(gen, len(lens), shape.num_q_heads, d)
    if kind == ha.HA_SWA:
        nr = len(lens) + 2
        ids = list(range(len(lens))) if ring_order is None else ring_order
        pool = ha.SwaRingPool(shape, nr, "cuda", fill=float("nan"))
        view = pool.view(i32(ids))
    else:
        rng = np.random.default_rng(table_perm_seed)
        per = [-(-n // shape.page_size) for n in lens]
        num_pages = sum(per) + 5
        perm = rng.permutation(num_pages)
        table = np.full((len(lens), max(per) + 1), -1, np.int32)
        off = 0
        for b, c in enumerate(per):
            table[b, :c] = perm[off:off + c]
            off += c
        pool = ha.FullPagePool(shape, num_pages, "cuda", fill=float("nan"))
        view = pool.view(i32(table))
    append_history(shape, view, seq, [0] * len(lens), lens if appended is None else appended)
    return seq, q, pool, view


def oracle_decode(shape, kind, seq, q, lens):
    outs, lses = [], []
    kname = "swa" if kind == ha.HA_SWA else "full"
    for b, n in enumerate(lens):
        if n == 0:
            outs.append(np.zeros((shape.num_q_heads, shape.head_dim)))
            lses.append(np.full(shape.num_q_heads, -np.inf))
            continue
        o, l = oracle_rows(host(q[b:b + 1]), host(seq[b][0][:n]), host(seq[b][1][:n]), [n - 1], kname,
                           shape.window, shape.softmax_scale or None)
        outs.append(o[0])
        lses.append(l[0])
    return np.stack(outs), np.stack(lses)


@pytest.mark.parametrize("kind", [ha.HA_SWA, ha.HA_FULL])
@pytest.mark.parametrize("hq,hkv,d,window", [(4, 1, 64, 128), (64, 8, 128, 128), (16, 16, 128, 32), (32, 2, 64, 64),
                                              (16, 2, 128, 256), (8, 8, 64, 512),
                                              # windows that are not a multiple of 16
                                              (8, 2, 64, 1), (8, 1, 64, 3), (16, 2, 128, 24), (32, 4, 64, 100)])
def test_decode_matches_oracle(kind, hq, hkv, d, window):
    shape = ha.HeadShape(hq, hkv, d, window=window)
    seq, q, pool, view = build(shape, kind, LENS, seed=hq * 7 + d)
    out, lse = ha.hybrid_attn_decode(shape, view, i32(LENS), q, max(LENS))
    torch.cuda.synchronize()
    ref_o, ref_l = oracle_decode(shape, kind, seq, q, LENS)
    assert_close(host(out), host(lse), ref_o, ref_l, f"kind={kind} shape={shape}")


@pytest.mark.parametrize("page_size", [32, 64, 256])
@pytest.mark.parametrize("splits", [0, 3, 40])
def test_decode_larger_pages(page_size, splits):
    """Pages of several 16-token blocks: a split may start and end inside a
    page, and the fused append writes the new token into the right block of
    its page."""
    shape = ha.HeadShape(16, 2, 128, page_size=page_size)
    seq, q, pool, view = build(shape, ha.HA_FULL, LENS, seed=61 + page_size)
    out, lse = ha.hybrid_attn_decode(shape, view, i32(LENS), q, max(LENS), num_splits=splits)
    _, _, pool_b, view_b = build(shape, ha.HA_FULL, LENS, seed=61 + page_size, appended=[n - 1 for n in LENS])
    k_new = torch.stack([seq[b][0][n - 1] for b, n in enumerate(LENS)]).contiguous()
    v_new = torch.stack([seq[b][1][n - 1] for b, n in enumerate(LENS)]).contiguous()
    ob, lb = ha.hybrid_attn_decode(shape, view_b, i32(LENS), q, max(LENS), num_splits=splits,
                                   k_new=k_new, v_new=v_new)
    torch.cuda.synchronize()
    ref_o, ref_l = oracle_decode(shape, ha.HA_FULL, seq, q, LENS)
    assert_close(host(out), host(lse), ref_o, ref_l, f"page_size={page_size} splits={splits}")
    assert torch.equal(out, ob) and torch.equal(lse, lb)
    assert torch.equal(pool.k.view(torch.int16), pool_b.k.view(torch.int16))
    assert torch.equal(pool.v.view(torch.int16), pool_b.v.view(torch.int16))


@pytest.mark.parametrize("splits", [1, 2, 3, 7, 40])
def test_decode_split_counts_agree(splits):
    shape = ha.HeadShape(64, 8, 128)
    lens = [5, 200, 3000, 4097]
    seq, q, pool, view = build(shape, ha.HA_FULL, lens, seed=5)
    # num_splits is a maximum: the blocks are divided into equal splits of
    # ceil(blocks / num_splits) blocks, which may need fewer splits.
    got = ha.hybrid_attn_decode_splits(shape, ha.HA_FULL, len(lens), max(lens), splits)
    assert got <= splits and (got == splits or splits > 8)
    out, lse = ha.hybrid_attn_decode(shape, view, i32(lens), q, max(lens), num_splits=splits)
    torch.cuda.synchronize()
    ref_o, ref_l = oracle_decode(shape, ha.HA_FULL, seq, q, lens)
    assert_close(host(out), host(lse), ref_o, ref_l, f"splits={splits}")


def test_filled_batch_with_one_long_sequence_splits():
    # 64 sequences x 8 kv heads give every CU two workgroups, but one sequence
    # is much longer than the rest: workgroups are capped at 1024 blocks, so
    # its keys still split (here in two), and the merge matches the oracle.
    shape = ha.HeadShape(64, 8, 128)
    lens = [3] * 40 + [17] * 22 + [600, 20000]
    assert ha.hybrid_attn_decode_splits(shape, ha.HA_FULL, len(lens), max(lens)) == 2
    seq, q, pool, view = build(shape, ha.HA_FULL, lens, seed=21)
    out, lse = ha.hybrid_attn_decode(shape, view, i32(lens), q, max(lens))
    torch.cuda.synchronize()
    ref_o, ref_l = oracle_decode(shape, ha.HA_FULL, seq, q, lens)
    assert_close(host(out), host(lse), ref_o, ref_l, "filled batch, one long sequence")


def test_empty_rows_and_float32_queries():
    shape = ha.HeadShape(4, 1, 64, softmax_scale=1.0 / 8.0)
    lens = [0, 40, 0, 129]
    for kind in (ha.HA_SWA, ha.HA_FULL):
        seq, q, pool, view = build(shape, kind, lens, seed=9)
        qf = q.float() + 1e-3          # float32 queries are rounded to bf16 by the library
        out, lse = ha.hybrid_attn_decode(shape, view, i32(lens), qf, max(lens))
        torch.cuda.synchronize()
        ref_o, ref_l = oracle_decode(shape, kind, seq, qf.to(torch.bfloat16), lens)
        o, l = host(out), host(lse)
        assert (o[[0, 2]] == 0).all() and np.isneginf(l[[0, 2]]).all()
        assert_close(o[[1, 3]], l[[1, 3]], ref_o[[1, 3]], ref_l[[1, 3]], f"kind={kind}")


def test_page_permutation_and_ring_id_invariance():
    shape = ha.HeadShape(64, 8, 128)
    lens = [17, 129, 1500]
    _, q, _, view_a = build(shape, ha.HA_FULL, lens, seed=3, table_perm_seed=1)
    _, _, _, view_b = build(shape, ha.HA_FULL, lens, seed=3, table_perm_seed=2)
    oa, la = ha.hybrid_attn_decode(shape, view_a, i32(lens), q, max(lens))
    ob, lb = ha.hybrid_attn_decode(shape, view_b, i32(lens), q, max(lens))
    _, _, _, ring_a = build(shape, ha.HA_SWA, lens, seed=3, ring_order=[0, 1, 2])
    _, _, _, ring_b = build(shape, ha.HA_SWA, lens, seed=3, ring_order=[4, 2, 0])
    ra, rla = ha.hybrid_attn_decode(shape, ring_a, i32(lens), q, max(lens))
    rb, rlb = ha.hybrid_attn_decode(shape, ring_b, i32(lens), q, max(lens))
    torch.cuda.synchronize()
    assert torch.equal(oa, ob) and torch.equal(la, lb)
    assert torch.equal(ra, rb) and torch.equal(rla, rlb)


def test_decode_is_deterministic():
    shape = ha.HeadShape(64, 8, 128)
    lens = [300, 5000]
    _, q, _, view = build(shape, ha.HA_FULL, lens, seed=4)
    o1, l1 = ha.hybrid_attn_decode(shape, view, i32(lens), q, max(lens))
    o2, l2 = ha.hybrid_attn_decode(shape, view, i32(lens), q, max(lens))
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


def test_workspace_reused_across_calls():
    """One caller-provided workspace serves consecutive split-K calls whose
    split counts differ per sequence and per call (stale partials of an
    earlier call are never merged into a later one)."""
    shape = ha.HeadShape(64, 8, 128)
    lens = [5, 200, 3000, 4097]
    seq, q, pool, view = build(shape, ha.HA_FULL, lens, seed=6)
    need = ha.hybrid_attn_workspace_size(shape, ha.HA_FULL, True, len(lens), max(lens), 7)
    ws = torch.full((need,), 0x7f, dtype=torch.uint8, device="cuda")   # poison: huge floats
    calls = [(lens, 7), ([4, 199, 1000, 4097], 7), ([5, 17, 3000, 2500], 3), (lens, 7)]
    for call_lens, splits in calls:
        out, lse = ha.hybrid_attn_decode(shape, view, i32(call_lens), q, max(lens), num_splits=splits,
                                         workspace=ws)
        torch.cuda.synchronize()
        ref_o, ref_l = oracle_decode(shape, ha.HA_FULL, seq, q, call_lens)
        assert_close(host(out), host(lse), ref_o, ref_l, f"lens={call_lens} splits={splits}")


def pool_bits(pool):
    return pool.k.view(torch.int16).clone(), pool.v.view(torch.int16).clone()


@pytest.mark.parametrize("kind", [ha.HA_SWA, ha.HA_FULL])
@pytest.mark.parametrize("hq,hkv,d,window,splits", [(64, 8, 128, 128, 0), (4, 1, 64, 32, 0), (64, 8, 128, 128, 7),
                                                      (32, 2, 64, 64, 3), (16, 2, 128, 256, 0),
                                                      (8, 2, 64, 24, 0), (8, 2, 64, 3, 0)])
def test_fused_append_equals_append_then_decode(kind, hq, hkv, d, window, splits):
    """Passing the new token's K/V appends it in the same launch: outputs and
    the pool afterwards are bit-identical to append-then-decode."""
    shape = ha.HeadShape(hq, hkv, d, window=window)
    seed = 40 + hq + d
    seq, q, pool_a, view_a = build(shape, kind, LENS, seed=seed)
    _, _, pool_b, view_b = build(shape, kind, LENS, seed=seed, appended=[n - 1 for n in LENS])
    k_new = torch.stack([seq[b][0][n - 1] for b, n in enumerate(LENS)]).contiguous()
    v_new = torch.stack([seq[b][1][n - 1] for b, n in enumerate(LENS)]).contiguous()
    oa, la = ha.hybrid_attn_decode(shape, view_a, i32(LENS), q, max(LENS), num_splits=splits)
    ob, lb = ha.hybrid_attn_decode(shape, view_b, i32(LENS), q, max(LENS), num_splits=splits,
                                   k_new=k_new, v_new=v_new)
    torch.cuda.synchronize()
    ref_o, ref_l = oracle_decode(shape, kind, seq, q, LENS)
    assert_close(host(ob), host(lb), ref_o, ref_l, f"fused kind={kind} shape={shape}")
    assert torch.equal(oa, ob) and torch.equal(la, lb)
    ka, va = pool_bits(pool_a)
    kb, vb = pool_bits(pool_b)
    assert torch.equal(ka, kb) and torch.equal(va, vb)


@pytest.mark.parametrize("kind", [ha.HA_SWA, ha.HA_FULL])
def test_fused_append_float32_sources_and_repeat(kind):
    """float32 q/k_new/v_new are rounded like the append calls round them, and
    repeating the fused call (the token is then already in the pool) is
    idempotent."""
    shape = ha.HeadShape(4, 1, 64, softmax_scale=1.0 / 8.0)
    lens = [1, 16, 17, 129, 300]
    seq, q, pool_a, view_a = build(shape, kind, lens, seed=12)
    _, _, pool_b, view_b = build(shape, kind, lens, seed=12, appended=[n - 1 for n in lens])
    k_new = torch.stack([seq[b][0][n - 1] for b, n in enumerate(lens)]).float().contiguous()
    v_new = torch.stack([seq[b][1][n - 1] for b, n in enumerate(lens)]).float().contiguous()
    oa, la = ha.hybrid_attn_decode(shape, view_a, i32(lens), q.float(), max(lens))
    for _ in range(2):
        ob, lb = ha.hybrid_attn_decode(shape, view_b, i32(lens), q.float(), max(lens), k_new=k_new, v_new=v_new)
        torch.cuda.synchronize()
        assert torch.equal(oa, ob) and torch.equal(la, lb)
        ka, va = pool_bits(pool_a)
        kb, vb = pool_bits(pool_b)
        assert torch.equal(ka, kb) and torch.equal(va, vb)
