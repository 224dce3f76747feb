"""Layer-wise restore of a reused prefix's KV from pinned host memory into the
pools, overlapped with prefill: the restored pools are bit-identical to pools
filled by direct appends of the same rows, the overlapped pipeline gives
bit-identical outputs to restore-then-prefill, and those outputs match the
oracle (max |O| error <= 1e-2, max |LSE| error <= 1e-3)."""

import numpy as np
import pytest
import torch

import hybrid_sliding_window_gqa_amd as ha
from gpu_util import assert_close, cu_from_counts, host, i32, make_generator, oracle_rows, randn_bf16
from hybrid_sliding_window_gqa_amd import group as grp

pytestmark = pytest.mark.gpu

REUSE = [300, 129, 1000, 0]     # reused prefix length L per sequence
NEW = [40, 20, 77, 33]          # new tokens after it


def setup(seed=3):
    shape = ha.HeadShape(16, 2, 128)
    b, w = len(REUSE), shape.window
    totals = [l + n for l, n in zip(REUSE, NEW)]
    per = [-(-t // 16) for t in totals]
    perm = np.random.default_rng(seed).permutation(sum(per) + 4)
    table = np.full((b, max(per)), -1, np.int32)
    off = 0
    for s, c in enumerate(per):
        table[s, :c] = perm[off:off + c]
        off += c

    def make_group():
        return grp.HybridGroup(shape, i32(list(range(b))), b, i32(table), len(perm), fill=float("nan"))

    gen = make_generator(seed)
    nl = len(grp.GROUP_KINDS)
    logical = [[(randn_bf16(gen, t, 2, 128), randn_bf16(gen, t, 2, 128), randn_bf16(gen, t, 16, 128))
                for t in totals] for _ in range(nl)]          # [layer][seq] = (k, v, q) over [0, total)
    first, counts, k_rows, v_rows = [], [], [], []
    for li, kind in enumerate(grp.GROUP_KINDS):
        f = [max(0, l - w) if kind == grp.SWA else 0 for l in REUSE]
        c = [l - x for l, x in zip(REUSE, f)]
        first.append(f)
        counts.append(c)
        k_rows.append(torch.cat([logical[li][s][0][f[s]:REUSE[s]] for s in range(b)]).contiguous())
        v_rows.append(torch.cat([logical[li][s][1][f[s]:REUSE[s]] for s in range(b)]).contiguous())
    return shape, make_group, logical, first, counts, k_rows, v_rows


def chunk_inputs(logical, li):
    cat = lambda j: torch.cat([logical[li][s][j][REUSE[s]:REUSE[s] + NEW[s]] for s in range(len(REUSE))]).contiguous()
    return cat(2), cat(0), cat(1)     # q, k_new, v_new


def prefill_plan(group, logical):
    qs, ks, vs, outs, lses = [], [], [], [], []
    t = sum(NEW)
    for li in range(len(group.layers)):
        q, k, v = chunk_inputs(logical, li)
        qs.append(q)
        ks.append(k)
        vs.append(v)
        outs.append(torch.empty(t, 16, 128, dtype=torch.float32, device="cuda"))
        lses.append(torch.empty(t, 16, dtype=torch.float32, device="cuda"))
    plan = grp.plan_prefill(group, qs, ks, vs, i32(REUSE), i32(cu_from_counts(NEW)), max(NEW), outs, lses)
    return plan, outs, lses


def test_restored_pools_equal_direct_appends():
    shape, make_group, logical, first, counts, k_rows, v_rows = setup()
    group, ref = make_group(), make_group()
    restore = grp.RestorePlan(group, grp.HostKv(group, first, counts, k_rows, v_rows))
    copy_stream = torch.cuda.Stream()
    restore.run(copy_stream)
    for li, layer in enumerate(ref.layers):
        fn = ha.swa_ring_append if layer.kind == grp.SWA else ha.full_pool_append
        fn(shape, layer.view, i32(first[li]), i32(cu_from_counts(counts[li])), k_rows[li], v_rows[li])
    torch.cuda.synchronize()
    for a, b in zip(group.layers, ref.layers):
        assert torch.equal(a.pool.k.view(torch.int16), b.pool.k.view(torch.int16)), a.kind
        assert torch.equal(a.pool.v.view(torch.int16), b.pool.v.view(torch.int16)), a.kind


def test_overlapped_pipeline_equals_serial_and_oracle():
    shape, make_group, logical, first, counts, k_rows, v_rows = setup(seed=4)
    compute, copy_stream = torch.cuda.current_stream(), torch.cuda.Stream()
    # serial: restore everything, then the prefill pass
    g1 = make_group()
    r1 = grp.RestorePlan(g1, grp.HostKv(g1, first, counts, k_rows, v_rows))
    p1, outs1, lses1 = prefill_plan(g1, logical)
    r1.run(copy_stream)
    torch.cuda.synchronize()
    p1.run(compute)
    torch.cuda.synchronize()
    # overlapped, twice in a row (the second run must not race the first)
    g2 = make_group()
    r2 = grp.RestorePlan(g2, grp.HostKv(g2, first, counts, k_rows, v_rows))
    p2, outs2, lses2 = prefill_plan(g2, logical)
    for _ in range(2):
        grp.run_restore_overlapped(r2, p2, compute, copy_stream)
    torch.cuda.synchronize()
    for li in range(len(g1.layers)):
        assert torch.equal(outs1[li], outs2[li]) and torch.equal(lses1[li], lses2[li]), f"layer {li}"
        for a, b in zip(g1.layers[li:li + 1], g2.layers[li:li + 1]):
            assert torch.equal(a.pool.k.view(torch.int16), b.pool.k.view(torch.int16))
    # the outputs against the oracle, an SWA layer and the full layer
    cu = cu_from_counts(NEW)
    for li in (0, len(g1.layers) - 1):
        kind = g1.layers[li].kind
        for s in range(len(REUSE)):
            k, v, q = logical[li][s]
            rows = np.arange(REUSE[s], REUSE[s] + NEW[s])
            ref_o, ref_l = oracle_rows(host(q)[rows], host(k), host(v), rows, kind, shape.window)
            assert_close(host(outs2[li])[cu[s]:cu[s + 1]], host(lses2[li])[cu[s]:cu[s + 1]], ref_o, ref_l,
                         f"layer {li} seq {s}")


def test_two_group_stack_sharing_staging():
    """Two groups restored on one copy stream through shared staging buffers,
    overlapped with their prefill passes: each group's outputs and pools equal
    those of a lone group restored and computed serially."""
    shape, make_group, logical, first, counts, k_rows, v_rows = setup(seed=5)
    compute, copy_stream = torch.cuda.current_stream(), torch.cuda.Stream()
    g0 = make_group()
    r0 = grp.RestorePlan(g0, grp.HostKv(g0, first, counts, k_rows, v_rows))
    p0, outs0, lses0 = prefill_plan(g0, logical)
    r0.run(copy_stream)
    torch.cuda.synchronize()
    p0.run(compute)
    torch.cuda.synchronize()
    groups = [make_group(), make_group()]
    host_kv = grp.HostKv(groups[0], first, counts, k_rows, v_rows)
    restores = [grp.RestorePlan(groups[0], host_kv)]
    restores.append(grp.RestorePlan(groups[1], host_kv, staging_from=restores[0]))
    assert restores[1].layers[-1][2] is restores[0].layers[-1][2]      # staging really shared
    plans = [prefill_plan(g, logical) for g in groups]
    grp.run_restore_overlapped(restores, [p for p, _, _ in plans], compute, copy_stream)
    torch.cuda.synchronize()
    for g, (_, outs, lses) in zip(groups, plans):
        for li in range(len(g.layers)):
            assert torch.equal(outs0[li], outs[li]) and torch.equal(lses0[li], lses[li]), f"layer {li}"
            assert torch.equal(g0.layers[li].pool.k.view(torch.int16), g.layers[li].pool.k.view(torch.int16))
            assert torch.equal(g0.layers[li].pool.v.view(torch.int16), g.layers[li].pool.v.view(torch.int16))
