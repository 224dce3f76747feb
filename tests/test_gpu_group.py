"""a9 on the GPU: a 6:1 layer group runs its calls in order (append then
attend for decode, or one fused call per layer; attend then append for
prefill), matches the oracle per layer, and replays bit-identically from a
captured HIP graph."""

import numpy as np
import pytest
import torch

import hybrid_sliding_window_gqa_amd as ha
from gpu_util import assert_close, cu_from_counts, host, i32, make_generator, oracle_rows, randn_bf16
from hybrid_sliding_window_gqa_amd import group as grp

pytestmark = pytest.mark.gpu


def setup_group(lens, shape, seed):
    b = len(lens)
    gen = make_generator(seed)
    per = [-(-(n + 1) // 16) for n in lens]
    num_pages = sum(per) + 4
    perm = np.random.default_rng(seed).permutation(num_pages)
    table = np.full((b, max(per)), -1, np.int32)
    off = 0
    for i, c in enumerate(per):
        table[i, :c] = perm[off:off + c]
        off += c
    group = grp.HybridGroup(shape, i32(list(range(b))[::-1]), b + 1, i32(table), num_pages, fill=float("nan"))
    hkv, hq, d = shape.num_kv_heads, shape.num_q_heads, shape.head_dim
    total = [n + 1 for n in lens]
    seqs = [[(randn_bf16(gen, t, hkv, d), randn_bf16(gen, t, hkv, d), randn_bf16(gen, t, hq, d)) for t in total]
            for _ in group.layers]
    return group, seqs


@pytest.mark.parametrize("fuse", [True, False])
def test_decode_step_order_oracle_and_graph_replay(fuse):
    shape = ha.HeadShape(16, 2, 128)
    lens = [5, 127, 128, 700, 1300]
    b = len(lens)
    group, seqs = setup_group(lens, shape, seed=8)
    # history: positions [0, n) of each sequence, per layer
    for li, layer in enumerate(group.layers):
        fn = ha.swa_ring_append if layer.kind == "swa" else ha.full_pool_append
        k = torch.cat([s[0][:n] for s, n in zip(seqs[li], lens)])
        v = torch.cat([s[1][:n] for s, n in zip(seqs[li], lens)])
        fn(shape, layer.view, i32([0] * b), i32(cu_from_counts(lens)), k, v)
    q = [torch.stack([s[2][n] for s, n in zip(seqs[li], lens)]).contiguous() for li in range(7)]
    kn = [torch.stack([s[0][n] for s, n in zip(seqs[li], lens)]).contiguous() for li in range(7)]
    vn = [torch.stack([s[1][n] for s, n in zip(seqs[li], lens)]).contiguous() for li in range(7)]
    out = [torch.empty(b, 16, 128, device="cuda") for _ in range(7)]
    lse = [torch.empty(b, 16, device="cuda") for _ in range(7)]
    plan = grp.plan_decode(group, q, kn, vn, i32(lens), i32([n + 1 for n in lens]), max(lens) + 1, out, lse,
                           fuse_append=fuse)
    if fuse:   # one call per layer appends the token and attends
        assert plan.labels == [f"decode[{i}:{k}]" for i, k in enumerate(grp.GROUP_KINDS)]
    else:
        assert plan.labels[:2] == ["append[0:swa]", "decode[0:swa]"] and plan.labels[-1] == "decode[6:full]"
    plan.run()
    torch.cuda.synchronize()
    eager = [(o.clone(), l.clone()) for o, l in zip(out, lse)]
    for li, layer in enumerate(group.layers):
        for bi, n in enumerate(lens):
            ref_o, ref_l = oracle_rows(host(q[li][bi:bi + 1]), host(seqs[li][bi][0]), host(seqs[li][bi][1]), [n],
                                       layer.kind, shape.window)
            assert_close(host(out[li][bi:bi + 1]), host(lse[li][bi:bi + 1]), ref_o, ref_l, f"layer {li} seq {bi}")

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=side):
        plan.run()
    torch.cuda.synchronize()
    for rep in range(4):
        for o in out:
            o.zero_()                      # eager work between replays
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for (eo, el), o, l in zip(eager, out, lse):
            assert torch.equal(eo, o) and torch.equal(el, l), f"replay {rep} differs from eager"


def test_prefill_chunk_plan_matches_oracle():
    shape = ha.HeadShape(16, 2, 128)
    lens = [40, 300, 129]
    b = len(lens)
    group, seqs = setup_group(lens, shape, seed=9)
    cut = [0, 100, 64]
    outs_all = [[None] * b for _ in range(7)]
    bounds = [([0] * b, cut), (cut, [n + 1 for n in lens])]
    for lo, hi in bounds:
        counts = [h - l for l, h in zip(lo, hi)]
        t = sum(counts)
        cat = lambda li, j: torch.cat([s[j][l:h] for s, l, h in zip(seqs[li], lo, hi)]).contiguous()
        q = [cat(li, 2) for li in range(7)]
        k = [cat(li, 0) for li in range(7)]
        v = [cat(li, 1) for li in range(7)]
        out = [torch.empty(t, 16, 128, device="cuda") for _ in range(7)]
        lse = [torch.empty(t, 16, device="cuda") for _ in range(7)]
        plan = grp.plan_prefill(group, q, k, v, i32(lo), i32(cu_from_counts(counts)), max(counts), out, lse)
        assert plan.labels[:2] == ["prefill[0:swa]", "append[0:swa]"]
        plan.run()
        torch.cuda.synchronize()
        cu = cu_from_counts(counts)
        for li in range(7):
            for bi in range(b):
                part = (host(out[li][cu[bi]:cu[bi + 1]]), host(lse[li][cu[bi]:cu[bi + 1]]))
                prev = outs_all[li][bi]
                outs_all[li][bi] = part if prev is None else (np.concatenate([prev[0], part[0]]),
                                                              np.concatenate([prev[1], part[1]]))
    for li, layer in enumerate(group.layers):
        for bi, n in enumerate(lens):
            pos = np.arange(n + 1)
            ref_o, ref_l = oracle_rows(host(seqs[li][bi][2]), host(seqs[li][bi][0]), host(seqs[li][bi][1]), pos,
                                       layer.kind, shape.window)
            assert_close(outs_all[li][bi][0], outs_all[li][bi][1], ref_o, ref_l, f"layer {li} seq {bi}")
