"""Helpers for the GPU parity tests: build pools from logical K/V through the
library's append calls, decode the documented pool layouts, and run the
oracle on the same logical tensors.

The oracle never sees anything the HIP path produced: its inputs are the
generator's logical Q/K/V (copied to the host), and only the outputs are
compared.
"""

from __future__ import annotations

import numpy as np
import torch

import hybrid_sliding_window_gqa_amd as ha
from oracle.attention import attend
from oracle.indexing import page_location, ring_contents

OUT_TOL = 1e-2
LSE_TOL = 1e-3
DEV = "cuda"


def i32(x, device=DEV):
    return torch.as_tensor(np.asarray(x, dtype=np.int32), device=device)


def cu_from_counts(counts):
    return np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)


def randn_bf16(gen, *shape):
    return torch.randn(*shape, generator=gen, device=DEV, dtype=torch.float32).to(torch.bfloat16)


def make_generator(seed):
    g = torch.Generator(device=DEV)
    g.manual_seed(seed)
    return g


def host(t):
    return t.detach().float().cpu().numpy()


def append_history(shape, view, seq_kv, starts, ends, src=None):
    """Append positions [starts[b], ends[b]) of each sequence's logical K/V
    (seq_kv[b] = (k [T_b, Hkv, D], v) device tensors) with one call."""
    counts = [int(e - s) for s, e in zip(starts, ends)]
    if sum(counts) == 0:
        return
    k_new = torch.cat([kv[0][s:e] for kv, s, e in zip(seq_kv, starts, ends)])
    v_new = torch.cat([kv[1][s:e] for kv, s, e in zip(seq_kv, starts, ends)])
    if src is not None:
        k_new, v_new = k_new.to(src), v_new.to(src)
    fn = ha.swa_ring_append if view.kind == ha.HA_SWA else ha.full_pool_append
    fn(shape, view, i32(starts), i32(cu_from_counts(counts)), k_new.contiguous(), v_new.contiguous())


def block_k(blocks, d):
    """Decode K blocks [..., 16*d] (the documented operand-order layout: value
    ((ch/32)*64 + ((ch%32)/8)*16 + t)*8 + ch%8) into [..., 16 tokens, d]."""
    a = np.asarray(blocks).reshape(*blocks.shape[:-1], d // 32, 4, 16, 8)   # a, q, token, j
    return np.moveaxis(a, -2, -4).reshape(*blocks.shape[:-1], 16, d)


def block_v(blocks, d):
    """Decode V blocks [..., 16*d] (value ((ch/32)*64 + (t/4)*16 + ch%16)*8 +
    ((ch%32)/16)*4 + t%4) into [..., 16 tokens, d]."""
    a = np.asarray(blocks).reshape(*blocks.shape[:-1], d // 32, 4, 16, 2, 4)   # a, q, c, h, r
    n = a.ndim
    order = list(range(n - 5)) + [n - 4, n - 1, n - 5, n - 2, n - 3]       # q, r, a, h, c
    return a.transpose(order).reshape(*blocks.shape[:-1], 16, d)


def ring_slots(pool: ha.SwaRingPool, ring, g):
    """Host copies of ring `ring`, kv head g: K [W, D], V [W, D] by slot."""
    d = pool.shape.head_dim
    return block_k(host(pool.k[ring, g]), d).reshape(-1, d), block_v(host(pool.v[ring, g]), d).reshape(-1, d)


def page_blocks(pool: ha.FullPagePool, g):
    """Host copies of every page of kv head g: K, V each [num_pages, page_size, D]."""
    d, ps = pool.shape.head_dim, pool.shape.page_size
    k = block_k(host(pool.k[:, g]), d).reshape(-1, ps, d)
    v = block_v(host(pool.v[:, g]), d).reshape(-1, ps, d)
    return k, v


def check_ring(pool, ring, seq_k, seq_v, appended_positions, window):
    """Ring contents equal the oracle ring model, bit-exact; untouched slots,
    and the last block's slots past W, stay NaN."""
    model = ring_contents(appended_positions, window)
    for g in range(seq_k.shape[1]):
        k, v = ring_slots(pool, ring, g)
        for s, p in enumerate(model):
            if p < 0:
                assert np.isnan(k[s]).all() and np.isnan(v[s]).all(), (ring, g, s)
            else:
                np.testing.assert_array_equal(k[s], seq_k[p, g])
                np.testing.assert_array_equal(v[s], seq_v[p, g])
        assert np.isnan(k[window:]).all() and np.isnan(v[window:]).all(), (ring, g, "padding slots")


def check_pages(pool, table_row, seq_k, seq_v, length):
    """Positions [0, length) sit at the oracle page model's (page, offset), bit-exact."""
    pos = np.arange(length)
    pages, offs = page_location(table_row, pos, pool.shape.page_size)
    for g in range(seq_k.shape[1]):
        k, v = page_blocks(pool, g)                  # [P, page_size, D] each
        np.testing.assert_array_equal(k[pages, offs], seq_k[:length, g])
        np.testing.assert_array_equal(v[pages, offs], seq_v[:length, g])


def oracle_rows(q_rows, k_seq, v_seq, positions, kind, window, scale=None):
    """Oracle output for query rows of one sequence (all host float arrays)."""
    return attend(q_rows, k_seq, v_seq, np.asarray(positions), kind, window, scale)


def assert_close(out, lse, ref_out, ref_lse, what=""):
    out = np.asarray(out)
    lse = np.asarray(lse)
    assert np.isfinite(out).all() and np.isfinite(lse).all(), f"non-finite output {what}"
    err_o = float(np.abs(out - ref_out).max()) if out.size else 0.0
    err_l = float(np.abs(lse - ref_lse).max()) if lse.size else 0.0
    assert err_o <= OUT_TOL, f"max |O - oracle| = {err_o:.3e} {what}"
    assert err_l <= LSE_TOL, f"max |LSE - oracle| = {err_l:.3e} {what}"
    return err_o, err_l
