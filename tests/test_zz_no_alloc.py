"""hybrid_attn_decode_noalloc (split-K partials in the library's static
scratch array) against hybrid_attn_decode with a caller workspace: the same
kernels and split counts, so the outputs must be bit-identical. Two calls in
a row, the second with a smaller input, so the second reads nothing the first
left behind; then one sampled row of each call against the oracle."""

import numpy as np
import pytest
import torch

import hybrid_sliding_window_gqa_amd as ha
from hybrid_sliding_window_gqa_amd import _lib
from gpu_util import DEV, OUT_TOL, LSE_TOL, append_history, host, i32, make_generator, oracle_rows, randn_bf16

pytestmark = pytest.mark.gpu


def _full_pool(shape, lens, seed):
    per = [-(-n // 16) for n in lens]
    perm = np.random.default_rng(seed).permutation(sum(per) + 5)
    table = np.full((len(lens), max(per)), -1, np.int32)
    off = 0
    for s, c in enumerate(per):
        table[s, :c] = perm[off:off + c]
        off += c
    pool = ha.FullPagePool(shape, len(perm), DEV, fill=float("nan"))
    return pool.view(i32(table))


def _case(shape, kind, lens, splits, seed):
    gen = make_generator(seed)
    hq, hkv, d = shape.num_q_heads, shape.num_kv_heads, shape.head_dim
    k = [randn_bf16(gen, n, hkv, d) for n in lens]
    v = [randn_bf16(gen, n, hkv, d) for n in lens]
    q = randn_bf16(gen, len(lens), hq, d)
    if kind == ha.HA_FULL:
        view = _full_pool(shape, lens, seed)
        starts = [0] * len(lens)
    else:
        pool = ha.SwaRingPool(shape, len(lens) + 2, DEV, fill=float("nan"))
        view = pool.view(i32(list(range(len(lens)))[::-1]))
        starts = [max(0, n - shape.window) for n in lens]
    append_history(shape, view, list(zip(k, v)), starts, lens)
    kv_len = i32(lens)
    print(f"[noalloc] kind={kind} lens={lens} splits={splits} "
          f"resolved={ha.hybrid_attn_decode_splits(shape, kind, len(lens), max(lens), splits)}", flush=True)
    ref_o, ref_l = ha.hybrid_attn_decode(shape, view, kv_len, q, max(lens), num_splits=splits)
    out = torch.full_like(ref_o, float("nan"))
    lse = torch.full_like(ref_l, float("nan"))
    ha.hybrid_attn_decode_noalloc(shape, view, kv_len, q, max(lens), out, lse, num_splits=splits)
    torch.cuda.synchronize()
    assert torch.equal(out, ref_o) and torch.equal(lse, ref_l)
    # one row against the oracle as well (the bar the decode parity tests use)
    s = int(np.argmax(lens))
    name = "full" if kind == ha.HA_FULL else "swa"
    o_ref, l_ref = oracle_rows(host(q[s:s + 1]), host(k[s]), host(v[s]), [lens[s] - 1], name, shape.window)
    assert float(np.abs(host(out[s:s + 1]) - o_ref).max()) <= OUT_TOL
    assert float(np.abs(host(lse[s:s + 1]) - l_ref).max()) <= LSE_TOL


def test_noalloc_equals_workspace_decode_twice_second_smaller():
    shape = ha.HeadShape(64, 8, 128)
    first = [3000, 5000, 777, 4096, 12345, 20]
    second = [1500, 33, 2049]
    assert ha.hybrid_attn_workspace_size(shape, ha.HA_FULL, True, len(first), max(first), 7) > \
        ha.hybrid_attn_workspace_size(shape, ha.HA_FULL, True, len(second), max(second), 5) > 0
    _case(shape, ha.HA_FULL, first, 7, seed=5)
    _case(shape, ha.HA_FULL, second, 5, seed=6)


def test_noalloc_automatic_splits_and_swa():
    shape = ha.HeadShape(64, 8, 128)
    lens = [30000, 9000]
    assert ha.hybrid_attn_decode_splits(shape, ha.HA_FULL, len(lens), max(lens)) > 1
    _case(shape, ha.HA_FULL, lens, 0, seed=7)
    _case(shape, ha.HA_SWA, [300, 5, 128], 0, seed=8)          # SWA: no partials at all
    _case(ha.HeadShape(4, 1, 64), ha.HA_FULL, [5000, 700], 3, seed=9)


def test_noalloc_rejects_partials_beyond_the_static_array():
    shape = ha.HeadShape(64, 8, 128)
    lens = [1 << 20] * 8
    assert ha.hybrid_attn_workspace_size(shape, ha.HA_FULL, True, 8, lens[0]) > _lib.HA_DECODE_SCRATCH_BYTES
    pool = ha.FullPagePool(shape, 4, DEV)
    view = pool.view(i32(np.zeros((8, 4), np.int32)))
    q = torch.zeros(8, 64, 128, dtype=torch.bfloat16, device=DEV)
    out = torch.empty(8, 64, 128, dtype=torch.float32, device=DEV)
    lse = torch.empty(8, 64, dtype=torch.float32, device=DEV)
    with pytest.raises(ha.HybridAttnError) as e:
        ha.hybrid_attn_decode_noalloc(shape, view, i32(lens), q, lens[0], out, lse)
    assert e.value.status == _lib.HA_ERR_WORKSPACE
