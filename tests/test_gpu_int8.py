"""INT8 KV pools on the GPU (include/hybrid_attn.h): the append calls write
exactly the oracle's codes and scales (oracle/quant.py) at the documented
byte positions, and decode over INT8 pools matches the oracle's attention
over the dequantized K/V (max |O| error <= 1e-2, max |LSE| error <= 1e-3)
across block, window and split edges, for bf16 and float32 inputs, up to the
full decode workload."""

import numpy as np
import pytest
import torch

import hybrid_sliding_window_gqa_amd as ha
import synth
from gpu_util import DEV, append_history, assert_close, host, i32, make_generator, randn_bf16
from hybrid_sliding_window_gqa_amd import group as grp
from oracle.attention import attend
from oracle.indexing import page_location, ring_contents
from oracle.quant import bf16_round, dequantize_rows, quantize_rows

pytestmark = pytest.mark.gpu


def k8_index(d):
    """[16, d] byte offsets of K(t, ch) in a block, as the header states them."""
    t, ch = np.meshgrid(np.arange(16), np.arange(d), indexing="ij")
    return ((ch // 64) * 64 + ((ch % 32) // 8) * 16 + t) * 16 + ((ch // 32) % 2) * 8 + ch % 8


def v8_index(d):
    t, ch = np.meshgrid(np.arange(16), np.arange(d), indexing="ij")
    return ((ch // 64) * 64 + (t // 4) * 16 + ch % 16) * 16 + ((ch // 16) % 4) * 4 + t % 4


def unpack(pool, d):
    """Host codes K, V [..., 16, d] (int) and scales [..., 16] of every block."""
    k = host(pool.k.view(torch.int8).to(torch.int32)).astype(np.int64)
    v = host(pool.v.view(torch.int8).to(torch.int32)).astype(np.int64)
    return (k[..., k8_index(d)], v[..., v8_index(d)], host(pool.k_scale), host(pool.v_scale))


def quantized(x_bf16_values):
    codes, scale = quantize_rows(x_bf16_values)
    return codes.astype(np.int64), scale


def make_pools(shape, kind, lens, seed=0):
    b = len(lens)
    if kind == ha.HA_SWA:
        pool = ha.SwaRingPool(shape, b + 1, DEV, fill=float("nan"), kv_dtype="int8")
        return pool, pool.view(i32(list(range(b))[::-1])), None
    per = [-(-max(n, 1) // shape.page_size) for n in lens]
    perm = np.random.default_rng(seed).permutation(sum(per) + 3)
    table = np.full((b, max(per)), -1, np.int32)
    off = 0
    for s, c in enumerate(per):
        table[s, :c] = perm[off:off + c]
        off += c
    pool = ha.FullPagePool(shape, len(perm), DEV, fill=float("nan"), kv_dtype="int8")
    return pool, pool.view(i32(table)), table


@pytest.mark.parametrize("kind", [ha.HA_SWA, ha.HA_FULL])
@pytest.mark.parametrize("d,window,src", [(128, 128, None), (64, 32, torch.float32), (128, 32, None),
                                          (64, 24, None), (64, 3, None)])
def test_append_writes_the_oracle_codes(kind, d, window, src):
    check_append_codes(kind, d, window, src, 16)


@pytest.mark.parametrize("page_size", [32, 64])
def test_append_codes_into_larger_pages(page_size):
    check_append_codes(ha.HA_FULL, 128, 128, None, page_size)


def check_append_codes(kind, d, window, src, page_size):
    shape = ha.HeadShape(8, 2, d, window=window, page_size=page_size)
    lens = [1, 15, 16, 17, 130, 300]
    gen = make_generator(3 + d + window)
    k = [randn_bf16(gen, n, 2, d) * 3 for n in lens]
    v = [randn_bf16(gen, n, 2, d) for n in lens]
    if src is not None:    # float32 values that are not bf16: rounded first
        k = [(x.float() + torch.randn(x.shape, generator=gen, device=DEV) * 1e-3) for x in k]
        v = [(x.float() + torch.randn(x.shape, generator=gen, device=DEV) * 1e-3) for x in v]
    k[0][:] = 0                                         # an all-zero row: scale 0, codes 0
    pool, view, table = make_pools(shape, kind, lens)
    # two calls: the first half, then the rest (rings keep only the last W)
    half = [n // 2 for n in lens]
    append_history(shape, view, list(zip(k, v)), [0] * len(lens), half)
    append_history(shape, view, list(zip(k, v)), half, lens)
    torch.cuda.synchronize()
    kc, vc, ks, vs = unpack(pool, d)
    for s, n in enumerate(lens):
        kx = bf16_round(host(k[s]))
        vx = bf16_round(host(v[s]))
        qk, sk = quantized(kx)                          # [n, hkv, d], [n, hkv]
        qv, sv = quantized(vx)
        for g in range(2):
            if kind == ha.HA_SWA:
                ring = len(lens) - 1 - s
                slots = ring_contents(list(range(n)), window)
                for slot, p in enumerate(slots):
                    blk, t = slot // 16, slot % 16
                    got = (kc[ring, g, blk, t], vc[ring, g, blk, t], ks[ring, g, blk, t], vs[ring, g, blk, t])
                    if p < 0:
                        assert np.all(got[0] == 127) and np.isnan(got[2]) and np.isnan(got[3])
                        continue
                    np.testing.assert_array_equal(got[0], qk[p, g])
                    np.testing.assert_array_equal(got[1], qv[p, g])
                    assert got[2] == sk[p, g] and got[3] == sv[p, g]
            else:
                # [pages, Hkv, page_size / 16, 16, ...] -> token offsets within a page
                kc, vc = (x.reshape(x.shape[0], x.shape[1], page_size, d) for x in (kc, vc))
                ks, vs = (x.reshape(x.shape[0], x.shape[1], page_size) for x in (ks, vs))
                pages, offs = page_location(table[s], np.arange(n), page_size)
                np.testing.assert_array_equal(kc[pages, g, offs], qk[:, g])
                np.testing.assert_array_equal(vc[pages, g, offs], qv[:, g])
                np.testing.assert_array_equal(ks[pages, g, offs], sk[:, g])
                np.testing.assert_array_equal(vs[pages, g, offs], sv[:, g])


def oracle_decode(q_row, k_seq, v_seq, n, kind, window):
    """Oracle for the query at position n - 1 over the dequantized K/V."""
    qk, sk = quantize_rows(bf16_round(k_seq[:n]))
    qv, sv = quantize_rows(bf16_round(v_seq[:n]))
    kd = np.stack([dequantize_rows(qk[:, g], sk[:, g]) for g in range(qk.shape[1])], axis=1)
    vd = np.stack([dequantize_rows(qv[:, g], sv[:, g]) for g in range(qv.shape[1])], axis=1)
    return attend(q_row[None], kd, vd, np.array([n - 1]), kind, window)


@pytest.mark.parametrize("kind", [ha.HA_SWA, ha.HA_FULL])
@pytest.mark.parametrize("hq,hkv,d,window,splits,qsrc", [(64, 8, 128, 128, 0, None), (16, 2, 64, 32, 3, None),
                                                          (32, 4, 128, 64, 7, torch.float32),
                                                          (8, 8, 128, 128, 1, None),
                                                          (16, 2, 64, 24, 0, None), (8, 2, 64, 3, 0, None)])
def test_decode_matches_oracle_over_dequantized_kv(kind, hq, hkv, d, window, splits, qsrc):
    check_decode(kind, hq, hkv, d, window, splits, qsrc, 16)


@pytest.mark.parametrize("page_size,splits", [(32, 0), (64, 3), (128, 40)])
def test_decode_over_larger_int8_pages(page_size, splits):
    check_decode(ha.HA_FULL, 16, 2, 128, 128, splits, None, page_size)


def check_decode(kind, hq, hkv, d, window, splits, qsrc, page_size):
    shape = ha.HeadShape(hq, hkv, d, window=window, page_size=page_size)
    lens = [1, 2, 15, 16, 17, window - 1, window, window + 1, 300, 1029, 2500]
    gen = make_generator(hq + d + window + splits)
    k = [randn_bf16(gen, n, hkv, d) for n in lens]
    v = [randn_bf16(gen, n, hkv, d) for n in lens]
    q = randn_bf16(gen, len(lens), hq, d)
    pool, view, _ = make_pools(shape, kind, lens, seed=hq)
    starts = [max(0, n - window) if kind == ha.HA_SWA else 0 for n in lens]
    append_history(shape, view, list(zip(k, v)), starts, lens)
    qq = q if qsrc is None else q.to(qsrc)
    out, lse = ha.hybrid_attn_decode(shape, view, i32(lens), qq, max(lens), num_splits=splits)
    torch.cuda.synchronize()
    kname = "swa" if kind == ha.HA_SWA else "full"
    for s, n in enumerate(lens):
        ref_o, ref_l = oracle_decode(host(q[s]), host(k[s]), host(v[s]), n, kname, window)
        assert_close(host(out[s:s + 1]), host(lse[s:s + 1]), ref_o, ref_l, f"kind={kind} len={n}")


def test_int8_decode_is_close_to_bf16_decode():
    """Quantization error on the output stays small next to bf16 pools."""
    shape = ha.HeadShape(64, 8, 128)
    lens = [300, 4000]
    gen = make_generator(9)
    k = [randn_bf16(gen, n, 8, 128) for n in lens]
    v = [randn_bf16(gen, n, 8, 128) for n in lens]
    q = randn_bf16(gen, len(lens), 64, 128)
    outs = []
    for fmt in ("bf16", "int8"):
        pool = ha.FullPagePool(shape, sum(-(-n // 16) for n in lens), DEV, kv_dtype=fmt)
        table = np.full((2, 250), -1, np.int32)
        table[0, :19] = np.arange(19)
        table[1, :250] = np.arange(19, 269)
        view = pool.view(i32(table))
        append_history(shape, view, list(zip(k, v)), [0, 0], lens)
        outs.append(host(ha.hybrid_attn_decode(shape, view, i32(lens), q, max(lens))[0]))
    torch.cuda.synchronize()
    assert np.abs(outs[0] - outs[1]).max() < 0.02


def test_decode_workload_with_int8_pools_sampled_sequences():
    """The decode workload's group (64 x 8192, 7 layers) on INT8 pools, one
    fused call per layer (quantize and append the token, attend); sampled
    sequences of every layer against the oracle."""
    struct = synth.decode_structure()
    shape = ha.HeadShape(struct.shape.num_q_heads, struct.shape.num_kv_heads, struct.shape.head_dim,
                         struct.shape.window)
    b, hist = struct.batch, int(struct.hist[0])
    hq, hkv, d, w = shape.num_q_heads, shape.num_kv_heads, shape.head_dim, shape.window
    group = grp.HybridGroup(shape, torch.as_tensor(struct.ring_id, device=DEV), struct.num_rings,
                            torch.as_tensor(struct.page_table, device=DEV), struct.num_pages, kv_dtype="int8")
    data = []
    for li, layer in enumerate(group.layers):
        lo = hist - (w - 1) if layer.kind == "swa" else 0
        n_hist = hist - lo
        k = synth.normal_bf16((b, n_hist + 1, hkv, d), "decode", li, synth.K_VALUES, DEV)
        v = synth.normal_bf16((b, n_hist + 1, hkv, d), "decode", li, synth.V_VALUES, DEV)
        q = synth.normal_bf16((b, hq, d), "decode", li, synth.Q_VALUES, DEV)
        fn = ha.swa_ring_append if layer.kind == "swa" else ha.full_pool_append
        fn(shape, layer.view, i32([lo] * b), i32(np.arange(b + 1) * n_hist),
           k[:, :n_hist].reshape(-1, hkv, d).contiguous(), v[:, :n_hist].reshape(-1, hkv, d).contiguous())
        data.append((k, v, q, lo))
    out = [torch.empty(b, hq, d, device=DEV) for _ in group.layers]
    lse = [torch.empty(b, hq, device=DEV) for _ in group.layers]
    plan = grp.plan_decode(group, [x[2] for x in data], [x[0][:, -1].contiguous() for x in data],
                           [x[1][:, -1].contiguous() for x in data], i32([hist] * b), i32([hist + 1] * b),
                           hist + 1, out, lse, fuse_append=True)
    plan.run()
    torch.cuda.synchronize()
    for li, layer in enumerate(group.layers):
        k, v, q, lo = data[li]
        for s in (0, 17, b - 1):
            ref_o, ref_l = oracle_decode(host(q[s]), host(k[s]), host(v[s]), hist - lo + 1, layer.kind, w)
            assert_close(host(out[li][s:s + 1]), host(lse[li][s:s + 1]), ref_o, ref_l, f"layer {li} seq {s}")


@pytest.mark.parametrize("kind", [ha.HA_SWA, ha.HA_FULL])
@pytest.mark.parametrize("d,window,qsrc", [(128, 128, None), (64, 32, torch.float32), (64, 24, None)])
def test_fused_append_equals_append_then_decode(kind, d, window, qsrc):
    """Decode with the new token's K/V quantizes and appends it in the same
    launch: pools and outputs bit-identical to append8 followed by decode."""
    shape = ha.HeadShape(16, 2, d, window=window)
    lens = [1, 2, 16, 17, window, window + 1, 300, 2049]
    gen = make_generator(d + window + kind)
    k = [randn_bf16(gen, n, 2, d) for n in lens]
    v = [randn_bf16(gen, n, 2, d) for n in lens]
    k[3][-1] = 0                                    # an all-zero new row: scale 0
    q = randn_bf16(gen, len(lens), 16, d)
    hist = [n - 1 for n in lens]
    starts = [max(0, h - window) if kind == ha.HA_SWA else 0 for h in hist]
    runs = []
    for fused in (True, False):
        pool, view, _ = make_pools(shape, kind, lens, seed=d)
        append_history(shape, view, list(zip(k, v)), starts, hist)
        k_new = torch.stack([x[-1] for x in k]).contiguous()
        v_new = torch.stack([x[-1] for x in v]).contiguous()
        if qsrc is not None:
            k_new, v_new = k_new.to(qsrc), v_new.to(qsrc)
        qq = q if qsrc is None else q.to(qsrc)
        if fused:
            out, lse = ha.hybrid_attn_decode(shape, view, i32(lens), qq, max(lens), k_new=k_new, v_new=v_new)
        else:
            fn = ha.swa_ring_append if kind == ha.HA_SWA else ha.full_pool_append
            fn(shape, view, i32(hist), i32(np.arange(len(lens) + 1)), k_new, v_new)
            out, lse = ha.hybrid_attn_decode(shape, view, i32(lens), qq, max(lens))
        torch.cuda.synchronize()
        runs.append((pool, host(out), host(lse)))
    (pa, oa, la), (pb, ob, lb) = runs
    assert torch.equal(pa.k, pb.k) and torch.equal(pa.v, pb.v)
    assert torch.equal(pa.k_scale.view(torch.int32), pb.k_scale.view(torch.int32))
    assert torch.equal(pa.v_scale.view(torch.int32), pb.v_scale.view(torch.int32))
    np.testing.assert_array_equal(oa, ob)
    np.testing.assert_array_equal(la, lb)


def test_int8_quantization_error_at_long_context():
    """The INT8 format's own error on the output at long context: decode of
    the full layer over INT8 pools against the oracle over the unquantized
    bf16 K/V, for the shortest, a middle and the longest sequence of the
    ragged long-context workload (1K to 1M cached tokens). Long sequences
    need the check most (blog.hotdry.top 2026-06-12, section "生产环境监控
    要点": sampled before/after-quantization checks, especially on long
    sequences). V's quantization alone moves O by at most half a step,
    max|V| / 254, per key; the bound allows one whole step."""
    shape = ha.HeadShape(64, 8, 128)
    hist = np.sort(synth.ragged_structure().hist.astype(np.int64))
    lens = [int(hist[0]) + 1, int(hist[len(hist) // 2]) + 1, int(hist[-1]) + 1]
    gen = make_generator(77)
    k = [randn_bf16(gen, n, 8, 128) for n in lens]
    v = [randn_bf16(gen, n, 8, 128) for n in lens]
    q = randn_bf16(gen, len(lens), 64, 128)
    pool, view, _ = make_pools(shape, ha.HA_FULL, lens, seed=5)
    append_history(shape, view, list(zip(k, v)), [0] * len(lens), lens)
    out, lse = ha.hybrid_attn_decode(shape, view, i32(lens), q, max(lens))
    torch.cuda.synchronize()
    for s, n in enumerate(lens):
        v_host = host(v[s])
        ref_o, ref_l = attend(host(q[s:s + 1]), host(k[s]), v_host, np.array([n - 1]), "full", shape.window)
        err_o = float(np.abs(host(out[s:s + 1]) - ref_o).max())
        err_l = float(np.abs(host(lse[s:s + 1]) - ref_l).max())
        v_max = float(np.abs(v_host).max())
        print(f"[int8 quantization error] {n} keys: max|O - oracle(bf16 K/V)| {err_o:.3e}, "
              f"max|LSE - oracle| {err_l:.3e} (max|V| {v_max:.2f})", flush=True)
        assert err_o <= v_max / 127 and err_l <= 1e-2, (n, err_o, err_l)


def oracle_rows8(q_rows, k_seq, v_seq, positions, kind, window):
    """Oracle rows at `positions` over the dequantized K/V of k_seq / v_seq."""
    qk, sk = quantize_rows(bf16_round(k_seq))
    qv, sv = quantize_rows(bf16_round(v_seq))
    kd = np.stack([dequantize_rows(qk[:, g], sk[:, g]) for g in range(qk.shape[1])], axis=1)
    vd = np.stack([dequantize_rows(qv[:, g], sv[:, g]) for g in range(qv.shape[1])], axis=1)
    return attend(q_rows, kd, vd, np.asarray(positions), kind, window)


@pytest.mark.parametrize("kind", [ha.HA_SWA, ha.HA_FULL])
@pytest.mark.parametrize("hq,hkv,d,window,nq,splits,src", [(64, 8, 128, 128, 4, 0, None),
                                                            (64, 8, 128, 128, 1, 3, None),
                                                            (8, 2, 64, 32, 8, 0, torch.float32),
                                                            (8, 4, 128, 24, 16, 5, None),
                                                            (8, 2, 64, 3, 4, 0, None)])
def test_verify_over_int8_pools(kind, hq, hkv, d, window, nq, splits, src):
    """Multi-token verify over INT8 pools: the nq new tokens are quantized as
    append8 does and attend, like the history, as codes times scales, so the
    rows match the oracle over the dequantized K/V of every position; the
    pool afterwards holds exactly the codes and scales of appending all
    tokens (bit-exact, including rows whose kv_len is below nq: nothing is
    written for them, and their outputs are 0 with LSE -inf)."""
    shape = ha.HeadShape(hq, hkv, d, window=window)
    lens = [nq, nq + 1, 17, window + nq, 300, 2049, max(nq - 1, 0)]
    gen = make_generator(hq + d + window + nq + splits)
    k = [randn_bf16(gen, max(n, nq), hkv, d) for n in lens]
    v = [randn_bf16(gen, max(n, nq), hkv, d) for n in lens]
    q = [randn_bf16(gen, max(n, nq), hq, d) for n in lens]
    hist = [max(n - nq, 0) for n in lens]
    pool, view, _ = make_pools(shape, kind, lens, seed=nq)
    ref_pool, ref_view, _ = make_pools(shape, kind, lens, seed=nq)
    starts = [max(0, h - window) if kind == ha.HA_SWA else 0 for h in hist]
    append_history(shape, view, list(zip(k, v)), starts, hist)
    rows = lambda xs: torch.stack([x[h:h + nq] for x, h in zip(xs, hist)]).contiguous()
    q_new, k_new, v_new = rows(q), rows(k), rows(v)
    if src is not None:
        q_new, k_new, v_new = q_new.to(src), k_new.to(src), v_new.to(src)
    out, lse = ha.hybrid_attn_verify(shape, view, i32(lens), q_new, k_new, v_new, max(lens), num_splits=splits)
    # reference pool: the history appended, then the nq tokens, by the append calls
    full_ends = [n if n >= nq else 0 for n in lens]
    append_history(shape, ref_view, list(zip(k, v)), starts, hist)
    fn = ha.swa_ring_append if kind == ha.HA_SWA else ha.full_pool_append
    live = [s for s, n in enumerate(lens) if n >= nq]
    fn(shape, ref_view, i32(hist), i32(np.concatenate([[0], np.cumsum([nq if n >= nq else 0 for n in lens])])),
       k_new[live].reshape(-1, hkv, d).contiguous(), v_new[live].reshape(-1, hkv, d).contiguous())
    torch.cuda.synchronize()
    kname = "swa" if kind == ha.HA_SWA else "full"
    o, l = host(out), host(lse)
    for s, n in enumerate(lens):
        if n < nq:
            assert np.all(o[s] == 0) and np.all(l[s] == -np.inf), f"row {s} (kv_len {n} < nq)"
            continue
        pos = np.arange(n - nq, n)
        ref_o, ref_l = oracle_rows8(host(q[s][n - nq:n]), host(k[s][:n]), host(v[s][:n]), pos, kname, window)
        assert_close(o[s], l[s], ref_o, ref_l, f"kind={kind} nq={nq} seq={s} len={n} full_end={full_ends[s]}")
    assert torch.equal(pool.k, ref_pool.k) and torch.equal(pool.v, ref_pool.v)
    assert torch.equal(pool.k_scale.view(torch.int32), ref_pool.k_scale.view(torch.int32))
    assert torch.equal(pool.v_scale.view(torch.int32), ref_pool.v_scale.view(torch.int32))
