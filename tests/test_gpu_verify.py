"""Multi-token verify decode on the GPU: nq new tokens per sequence, causal
among themselves, over ring and page pools, match the oracle (max |O| error
<= 1e-2, max |LSE| error <= 1e-3) for ragged lengths that span block, window
and split edges; equal prefill of an nq-token chunk and, for nq = 1, the
fused-append decode; leave the pool exactly as appending the tokens would."""

import numpy as np
import pytest
import torch

import hybrid_sliding_window_gqa_amd as ha
from gpu_util import append_history, assert_close, host, i32, make_generator, oracle_rows, randn_bf16

pytestmark = pytest.mark.gpu

# total lengths kv_len (history = kv_len - nq): short rows, rows whose new
# tokens straddle a 16-token block, window edges, several full-layer splits
LENS = [4, 5, 14, 18, 31, 130, 131, 300, 1000, 2051]


def make_pool(shape, kind, lens, perm_seed=0):
    b = len(lens)
    if kind == ha.HA_SWA:
        pool = ha.SwaRingPool(shape, b + 2, "cuda", fill=float("nan"))
        return pool, pool.view(i32(list(range(b))[::-1]))
    per = [-(-max(n, 1) // shape.page_size) for n in lens]
    num_pages = sum(per) + 5
    perm = np.random.default_rng(perm_seed).permutation(num_pages)
    table = np.full((b, max(per) + 1), -1, np.int32)
    off = 0
    for i, c in enumerate(per):
        table[i, :c] = perm[off:off + c]
        off += c
    pool = ha.FullPagePool(shape, num_pages, "cuda", fill=float("nan"))
    return pool, pool.view(i32(table))


class Case:
    """Per sequence: K/V/Q for positions [0, kv_len); the pool holds the
    history [0, kv_len - nq)."""

    def __init__(self, shape, kind, lens, nq, seed, src=None):
        gen = make_generator(seed)
        hq, hkv, d = shape.num_q_heads, shape.num_kv_heads, shape.head_dim
        self.shape, self.kind, self.lens, self.nq = shape, kind, lens, nq
        self.k = [randn_bf16(gen, max(n, nq), hkv, d) for n in lens]
        self.v = [randn_bf16(gen, max(n, nq), hkv, d) for n in lens]
        self.q = [randn_bf16(gen, max(n, nq), hq, d) for n in lens]
        self.pool, self.view = make_pool(shape, kind, lens)
        self.hist = [max(n - nq, 0) for n in lens]
        append_history(shape, self.view, list(zip(self.k, self.v)), [0] * len(lens), self.hist)
        rows = lambda xs: torch.stack([x[h:h + nq] for x, h in zip(xs, self.hist)]).contiguous()
        self.q_new, self.k_new, self.v_new = rows(self.q), rows(self.k), rows(self.v)
        if src is not None:
            self.q_new, self.k_new, self.v_new = (t.to(src) for t in (self.q_new, self.k_new, self.v_new))

    def run(self, num_splits=0):
        out, lse = ha.hybrid_attn_verify(self.shape, self.view, i32(self.lens), self.q_new, self.k_new, self.v_new,
                                         max(self.lens), num_splits=num_splits)
        torch.cuda.synchronize()
        return host(out), host(lse)

    def oracle(self):
        kname = "swa" if self.kind == ha.HA_SWA else "full"
        outs, lses = [], []
        for b, n in enumerate(self.lens):
            if n < self.nq:
                outs.append(np.zeros((self.nq, self.shape.num_q_heads, self.shape.head_dim)))
                lses.append(np.full((self.nq, self.shape.num_q_heads), -np.inf))
                continue
            pos = np.arange(n - self.nq, n)
            o, l = oracle_rows(host(self.q[b][n - self.nq:n]), host(self.k[b][:n]), host(self.v[b][:n]), pos, kname,
                               self.shape.window, self.shape.softmax_scale or None)
            outs.append(o)
            lses.append(l)
        return np.stack(outs), np.stack(lses)


def check(case, out, lse):
    ref_o, ref_l = case.oracle()
    for b, n in enumerate(case.lens):
        if n < case.nq:
            assert np.all(out[b] == 0) and np.all(lse[b] == -np.inf), f"row {b} (kv_len {n} < nq)"
        else:
            assert_close(out[b], lse[b], ref_o[b], ref_l[b], f"kind={case.kind} nq={case.nq} seq={b} len={n}")


@pytest.mark.parametrize("kind", [ha.HA_SWA, ha.HA_FULL])
@pytest.mark.parametrize("hq,hkv,d,window,nq", [(64, 8, 128, 128, 4), (64, 8, 128, 128, 1), (64, 8, 128, 128, 3),
                                                 (4, 1, 64, 128, 8), (16, 16, 128, 32, 16), (32, 2, 64, 64, 2),
                                                 (16, 16, 64, 16, 16), (16, 8, 64, 48, 8),
                                                 # windows that are not a multiple of 16, some below nq
                                                 (8, 2, 64, 3, 4), (8, 1, 64, 1, 2), (16, 2, 128, 24, 4),
                                                 (32, 4, 64, 100, 3)])
def test_verify_matches_oracle_and_appends(kind, hq, hkv, d, window, nq):
    shape = ha.HeadShape(hq, hkv, d, window=window)
    lens = [n for n in LENS] + [nq - 1 if nq > 1 else 0]     # one row shorter than nq
    case = Case(shape, kind, lens, nq, seed=hq + 3 * nq + d)
    out, lse = case.run()
    check(case, out, lse)
    # the pool now equals one that had every token appended
    ref_pool, ref_view = make_pool(shape, kind, lens)
    append_history(shape, ref_view, list(zip(case.k, case.v)), [0] * len(lens),
                   [n if n >= nq else 0 for n in lens])
    torch.cuda.synchronize()
    assert torch.equal(case.pool.k.view(torch.int16), ref_pool.k.view(torch.int16))
    assert torch.equal(case.pool.v.view(torch.int16), ref_pool.v.view(torch.int16))


@pytest.mark.parametrize("page_size,nq,splits", [(32, 4, 0), (64, 7, 3), (256, 16, 40)])
def test_verify_over_larger_pages(page_size, nq, splits):
    # the new tokens start inside a page of several 16-token blocks, and
    # splits start and end inside pages (group 2: nq x group <= 32)
    shape = ha.HeadShape(8, 4, 128, page_size=page_size)
    case = Case(shape, ha.HA_FULL, LENS, nq, seed=page_size + nq)
    out, lse = case.run(num_splits=splits)
    check(case, out, lse)
    ref_pool, ref_view = make_pool(shape, ha.HA_FULL, LENS)
    append_history(shape, ref_view, list(zip(case.k, case.v)), [0] * len(LENS), [n if n >= nq else 0 for n in LENS])
    torch.cuda.synchronize()
    assert torch.equal(case.pool.k.view(torch.int16), ref_pool.k.view(torch.int16))
    assert torch.equal(case.pool.v.view(torch.int16), ref_pool.v.view(torch.int16))


@pytest.mark.parametrize("splits", [1, 2, 5, 40])
def test_verify_split_counts_agree(splits):
    shape = ha.HeadShape(64, 8, 128)
    lens = [6, 300, 3001, 4100]
    case = Case(shape, ha.HA_FULL, lens, 4, seed=11)
    out, lse = case.run(num_splits=splits)
    check(case, out, lse)


@pytest.mark.parametrize("kind", [ha.HA_SWA, ha.HA_FULL])
def test_verify_equals_prefill_of_the_chunk_and_float32_inputs(kind):
    shape = ha.HeadShape(64, 8, 128)
    lens = [9, 140, 700]
    nq = 4
    case = Case(shape, kind, lens, nq, seed=5)
    # prefill of the same nq-token chunks, on a pool that holds only the history
    pre = Case(shape, kind, lens, nq, seed=5)
    cu = i32(np.arange(len(lens) + 1) * nq)
    flat = lambda t: t.reshape(len(lens) * nq, *t.shape[2:]).contiguous()
    p_out, p_lse = ha.hybrid_attn_prefill(shape, pre.view, i32(pre.hist), cu, flat(pre.q_new), flat(pre.k_new),
                                          flat(pre.v_new), max_new=nq)
    torch.cuda.synchronize()
    out, lse = case.run()
    assert np.abs(out.reshape(-1, 64, 128) - host(p_out)).max() <= 1e-2
    assert np.abs(lse.reshape(-1, 64) - host(p_lse)).max() <= 1e-3
    f32 = Case(shape, kind, lens, nq, seed=5, src=torch.float32)
    out32, lse32 = f32.run()
    check(f32, out32, lse32)


@pytest.mark.parametrize("kind", [ha.HA_SWA, ha.HA_FULL])
def test_verify_one_token_equals_fused_decode(kind):
    shape = ha.HeadShape(64, 8, 128)
    lens = [1, 17, 129, 1000]
    a = Case(shape, kind, lens, 1, seed=8)
    b = Case(shape, kind, lens, 1, seed=8)
    out, lse = a.run()
    d_out, d_lse = ha.hybrid_attn_decode(shape, b.view, i32(lens), b.q_new[:, 0].contiguous(), max(lens),
                                         k_new=b.k_new[:, 0].contiguous(), v_new=b.v_new[:, 0].contiguous())
    torch.cuda.synchronize()
    assert np.abs(out[:, 0] - host(d_out)).max() <= 1e-2
    assert np.abs(lse[:, 0] - host(d_lse)).max() <= 1e-3
    assert torch.equal(a.pool.k.view(torch.int16), b.pool.k.view(torch.int16))
    assert torch.equal(a.pool.v.view(torch.int16), b.pool.v.view(torch.int16))


def test_swa_verify_with_ring_holding_only_the_needed_window():
    """The ring only has to hold [t0 - W + 1, t0): the slot of t0 - W holds
    NaN here and must not reach the output."""
    shape = ha.HeadShape(64, 8, 128)
    lens, nq, w = [304, 132, 1004], 4, 128
    gen = make_generator(71)
    k = [randn_bf16(gen, n, 8, 128) for n in lens]
    v = [randn_bf16(gen, n, 8, 128) for n in lens]
    q = [randn_bf16(gen, n, 64, 128) for n in lens]
    pool = ha.SwaRingPool(shape, len(lens), "cuda", fill=float("nan"))
    view = pool.view(i32(list(range(len(lens)))))
    t0 = [n - nq for n in lens]
    append_history(shape, view, list(zip(k, v)), [t - (w - 1) for t in t0], t0)
    rows = lambda xs: torch.stack([x[t:t + nq] for x, t in zip(xs, t0)]).contiguous()
    out, lse = ha.hybrid_attn_verify(shape, view, i32(lens), rows(q), rows(k), rows(v), max(lens))
    torch.cuda.synchronize()
    for b, n in enumerate(lens):
        pos = np.arange(n - nq, n)
        ref_o, ref_l = oracle_rows(host(q[b][n - nq:n]), host(k[b]), host(v[b]), pos, "swa", w)
        assert_close(host(out[b]), host(lse[b]), ref_o, ref_l, f"seq {b}")
