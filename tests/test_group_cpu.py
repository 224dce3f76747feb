"""Host logic of the layer-group plans: a plan holds every tensor whose
address it passes to the library, so a caller may drop its own references
(the plans are built here on CPU tensors and never run)."""

import gc
import weakref

import torch

import hybrid_sliding_window_gqa_amd as ha
from hybrid_sliding_window_gqa_amd import group as grp


def small_group(b=2):
    shape = ha.HeadShape(8, 2, 64, window=32)
    ring = torch.arange(b, dtype=torch.int32)
    table = torch.arange(b * 4, dtype=torch.int32).reshape(b, 4)
    return shape, grp.HybridGroup(shape, ring, b, table, b * 4)


def test_prefill_plan_holds_its_tensors():
    shape, group = small_group()
    nl, t = len(group.layers), 5
    q = [torch.zeros(t, 8, 64, dtype=torch.bfloat16) for _ in range(nl)]
    k = [torch.zeros(t, 2, 64, dtype=torch.bfloat16) for _ in range(nl)]
    v = [torch.zeros(t, 2, 64, dtype=torch.bfloat16) for _ in range(nl)]
    out = [torch.empty(t, 8, 64) for _ in range(nl)]
    lse = [torch.empty(t, 8) for _ in range(nl)]
    hist = torch.tensor([3, 0], dtype=torch.int32)
    cu = torch.tensor([0, 2, 5], dtype=torch.int32)
    plan = grp.plan_prefill(group, q, k, v, hist, cu, 3, out, lse)
    refs = [weakref.ref(x) for x in q + k + v + out + lse + [hist, cu]]
    refs += [weakref.ref(layer.pool.k) for layer in group.layers]
    del q, k, v, out, lse, hist, cu, group
    gc.collect()
    assert all(r() is not None for r in refs)
    del plan
    gc.collect()
    assert all(r() is None for r in refs)


def decode_plan_refs(fuse):
    shape, group = small_group()
    nl, b = len(group.layers), 2
    q = [torch.zeros(b, 8, 64, dtype=torch.bfloat16) for _ in range(nl)]
    k = [torch.zeros(b, 2, 64, dtype=torch.bfloat16) for _ in range(nl)]
    v = [torch.zeros(b, 2, 64, dtype=torch.bfloat16) for _ in range(nl)]
    out = [torch.empty(b, 8, 64) for _ in range(nl)]
    lse = [torch.empty(b, 8) for _ in range(nl)]
    pos = torch.tensor([4, 9], dtype=torch.int32)
    kv_len = pos + 1
    plan = grp.plan_decode(group, q, k, v, pos, kv_len, 10, out, lse, fuse_append=fuse)
    refs = [weakref.ref(x) for x in q + k + v + out + lse + [pos, kv_len]]
    return plan, refs


def test_decode_plan_holds_its_tensors():
    for fuse in (True, False):
        plan, refs = decode_plan_refs(fuse)
        gc.collect()
        assert all(r() is not None for r in refs), fuse
        del plan
        gc.collect()
        assert all(r() is None for r in refs), fuse


def test_group_copies_share_a_pool_and_the_swa_pool_is_o_of_w():
    shape, group = small_group()
    full_i = group.kinds.index("full")
    ring = torch.arange(2, dtype=torch.int32)
    table = torch.arange(8, dtype=torch.int32).reshape(2, 4)
    copy = grp.HybridGroup(shape, ring, 2, table, 8, pools={full_i: group.layers[full_i].pool})
    assert copy.layers[full_i].pool is group.layers[full_i].pool
    assert all(copy.layers[i].pool is not group.layers[i].pool for i in range(len(group.layers)) if i != full_i)
    # 6 SWA layers x 2 rings x W slots x Hkv * D * 2 (K, V) * 2 bytes, whatever the history length
    assert group.pool_bytes()["swa"] == 6 * 2 * shape.window * shape.num_kv_heads * shape.head_dim * 4
    try:
        grp.HybridGroup(shape, ring, 2, table, 8, pools={0: group.layers[full_i].pool})
    except ValueError:
        pass
    else:
        raise AssertionError("a Full pool was accepted for an SWA layer")


def test_verify_plan_holds_its_tensors():
    shape, group = small_group()
    nl, nq = len(group.layers), 3
    q = [torch.zeros(2, nq, 8, 64, dtype=torch.bfloat16) for _ in range(nl)]
    k = [torch.zeros(2, nq, 2, 64, dtype=torch.bfloat16) for _ in range(nl)]
    v = [torch.zeros(2, nq, 2, 64, dtype=torch.bfloat16) for _ in range(nl)]
    out = [torch.empty(2, nq, 8, 64) for _ in range(nl)]
    lse = [torch.empty(2, nq, 8) for _ in range(nl)]
    kv_len = torch.tensor([10, 40], dtype=torch.int32)
    refs = [weakref.ref(t) for t in q + k + v + out + lse]
    plan = grp.plan_verify(group, q, k, v, kv_len, 40, out, lse)
    del q, k, v, out, lse
    gc.collect()
    assert all(r() is not None for r in refs)
    assert len(plan.calls) == nl and plan.labels[-1] == f"verify[{nl - 1}:full]"
