"""Page-table entries that name no page (-1, or an id past the pool) inside
a sequence's history: decode, verify and prefill all treat the 16 positions
of such a block as missing keys, and the appends drop their writes to it.
The oracle for that is plain attention over the positions that remain
(a full layer sees every earlier key, so removing keys only renumbers them);
an out-of-range ring id leaves a sequence without history keys."""

import numpy as np
import pytest
import torch

import hybrid_sliding_window_gqa_amd as ha
from gpu_util import DEV, LSE_TOL, OUT_TOL, append_history, assert_close, cu_from_counts, host, i32
from gpu_util import make_generator, randn_bf16
from oracle.attention import attend

pytestmark = pytest.mark.gpu

SHAPE = ha.HeadShape(64, 8, 128)
BAD_BLOCKS = {0: [3, 10], 1: [0], 2: []}       # per sequence: history blocks without a page


def setup(hist, new):
    totals = [h + n for h, n in zip(hist, new)]
    gen = make_generator(51)
    hkv, d = SHAPE.num_kv_heads, SHAPE.head_dim
    k = [randn_bf16(gen, t, hkv, d) for t in totals]
    v = [randn_bf16(gen, t, hkv, d) for t in totals]
    per = [-(-t // 16) for t in totals]
    num_pages = sum(per) + 4
    perm = np.random.default_rng(52).permutation(num_pages)
    table = np.full((len(totals), max(per)), -1, np.int32)
    off = 0
    for b, c in enumerate(per):
        table[b, :c] = perm[off:off + c]
        off += c
        for j, blk in enumerate(BAD_BLOCKS[b]):
            table[b, blk] = -1 if j % 2 == 0 else num_pages + 100     # no page / an id past the pool
    pool = ha.FullPagePool(SHAPE, num_pages, DEV, fill=float("nan"))
    view = pool.view(i32(table))
    append_history(SHAPE, view, list(zip(k, v)), [0] * len(totals), hist)
    return k, v, view, totals


def kept_positions(b, total):
    keep = np.ones(total, bool)
    for blk in BAD_BLOCKS[b]:
        keep[16 * blk:16 * blk + 16] = False
    return np.nonzero(keep)[0]


def test_prefill_and_decode_skip_blocks_without_a_page():
    hist, new = [700, 40, 333], [50, 17, 64]
    k, v, view, totals = setup(hist, new)
    gen = make_generator(53)
    q = randn_bf16(gen, sum(new), SHAPE.num_q_heads, SHAPE.head_dim)
    cat = lambda xs: torch.cat([x[h:t] for x, h, t in zip(xs, hist, totals)]).contiguous()
    cu = cu_from_counts(new)
    out, lse = ha.hybrid_attn_prefill(SHAPE, view, i32(hist), i32(cu), q, cat(k), cat(v), max_new=max(new))
    torch.cuda.synchronize()
    o, l = host(out), host(lse)
    for b in range(len(hist)):
        keep = kept_positions(b, totals[b])
        kk, vv = host(k[b])[keep], host(v[b])[keep]
        rows = np.searchsorted(keep, np.arange(hist[b], totals[b]))     # the queries' renumbered positions
        ref_o, ref_l = attend(host(q[cu[b]:cu[b + 1]]), kk, vv, rows, "full", SHAPE.window)
        assert_close(o[cu[b]:cu[b + 1]], l[cu[b]:cu[b + 1]], ref_o, ref_l, f"prefill seq {b}")
    # decode of position hist (appended in the same call) over the same table
    qd = randn_bf16(gen, len(hist), SHAPE.num_q_heads, SHAPE.head_dim)
    kn = torch.stack([k[b][hist[b]] for b in range(len(hist))]).contiguous()
    vn = torch.stack([v[b][hist[b]] for b in range(len(hist))]).contiguous()
    lens = [h + 1 for h in hist]
    for splits in (1, 5):
        out, lse = ha.hybrid_attn_decode(SHAPE, view, i32(lens), qd, max(lens), num_splits=splits, k_new=kn,
                                         v_new=vn)
        torch.cuda.synchronize()
        for b in range(len(hist)):
            keep = kept_positions(b, lens[b])
            ref_o, ref_l = attend(host(qd[b:b + 1]), host(k[b])[keep], host(v[b])[keep], [len(keep) - 1], "full",
                                  SHAPE.window)
            assert_close(host(out[b:b + 1]), host(lse[b:b + 1]), ref_o, ref_l, f"decode seq {b} splits {splits}")


def test_decode_with_an_invalid_ring_id_has_no_keys():
    pool = ha.SwaRingPool(SHAPE, 2, DEV, fill=float("nan"))
    view = pool.view(i32([0, 7]))                      # sequence 1 names a ring past the pool
    gen = make_generator(54)
    k, v = randn_bf16(gen, 300, 8, 128), randn_bf16(gen, 300, 8, 128)
    append_history(SHAPE, pool.view(i32([0, 1])), [(k, v), (k, v)], [0, 0], [300, 300])
    q = randn_bf16(gen, 2, 64, 128)
    out, lse = ha.hybrid_attn_decode(SHAPE, view, i32([300, 300]), q, 300)
    torch.cuda.synchronize()
    o, l = host(out), host(lse)
    ref_o, ref_l = attend(host(q[0:1]), host(k), host(v), [299], "swa", SHAPE.window)
    assert np.abs(o[0] - ref_o[0]).max() <= OUT_TOL and np.abs(l[0] - ref_l[0]).max() <= LSE_TOL
    assert (o[1] == 0).all() and np.isneginf(l[1]).all()
