"""The five synthetic workloads at full size, in the launch configuration the
bench uses (7-layer 6:1 groups through the step plans), checked against the
fp64 oracle on sampled rows (bf16 inputs, fp32 accumulation: max |O| error
<= 1e-2, max |LSE| error <= 1e-3).

  small    1 x 512 tokens, SWA + full layer, Hq/Hkv/D 4/1/64, float32 inputs:
           one-shot and 4 x 128-chunk prefill, then 16 decode steps; all rows.
  decode   64 sequences x 8192 cached tokens, one decode step; all rows.
  chunked  4 x 32768 tokens in 8192-token chunks; stratified row sample.
  reuse    32 ragged prefix-reuse requests (window-safe length from the
           library, checked against the oracle's brute force), ring restored
           from the cached window; plus the false-hit case: reusing the full
           token match restores evicted (NaN) slots and produces NaN rows.
  ragged   24 sequences up to 1M cached tokens, one decode step with split-K;
           SWA rows for all, full-layer rows for a sample of sequences.
  verify   the decode workload's shapes with 4 new tokens per sequence per
           layer through hybrid_attn_verify; all rows.
"""

import numpy as np
import pytest
import torch

import hybrid_sliding_window_gqa_amd as ha
import synth
from gpu_util import assert_close, cu_from_counts, host, i32
from hybrid_sliding_window_gqa_amd import group as grp
from oracle.attention import attend
from oracle.window_safe import window_safe_length

pytestmark = pytest.mark.gpu
DEV = "cuda"


def head_shape(struct, scale=0.0):
    s = struct.shape
    return ha.HeadShape(s.num_q_heads, s.num_kv_heads, s.head_dim, s.window, softmax_scale=scale)


def make_group(struct, shape, fill=None):
    return grp.HybridGroup(shape, i32(struct.ring_id), struct.num_rings, i32(struct.page_table),
                           struct.num_pages, fill=fill)


def seq_values(workload, layer, total, hkv, hq, d):
    """Logical K, V [total, Hkv, D] and Q [total, Hq, D] of one layer (all sequences concatenated)."""
    k = synth.normal_bf16((total, hkv, d), workload, layer, synth.K_VALUES, DEV)
    v = synth.normal_bf16((total, hkv, d), workload, layer, synth.V_VALUES, DEV)
    q = synth.normal_bf16((total, hq, d), workload, layer, synth.Q_VALUES, DEV)
    return k, v, q


def append_rows(shape, layer, pos0, k_rows, v_rows, counts):
    fn = ha.swa_ring_append if layer.kind == "swa" else ha.full_pool_append
    fn(shape, layer.view, i32(pos0), i32(cu_from_counts(counts)), k_rows.contiguous(), v_rows.contiguous())


def check_rows(shape, kind, q_rows, k_seq, v_seq, positions, out, lse, what, scale=None):
    ref_o, ref_l = attend(q_rows, k_seq, v_seq, positions, kind, shape.window, scale)
    return assert_close(out, lse, ref_o, ref_l, what)


def check_rows_dev(shape, kind, q_dev, k_dev, v_dev, rows, out, lse, what):
    """Oracle check of rows `rows` of one sequence whose logical K/V/Q live on
    the device. SWA rows are checked one window at a time (the window mask
    only depends on t - j), so only the keys a row can see are copied."""
    rows = np.asarray(rows)
    if kind == "full":
        last = int(rows.max()) + 1
        check_rows(shape, kind, host(q_dev[torch.as_tensor(rows, device=DEV)]), host(k_dev[:last]),
                   host(v_dev[:last]), rows, out, lse, what)
        return
    w = shape.window
    for i, r in enumerate(rows.tolist()):
        lo = max(0, r - w + 1)
        check_rows(shape, kind, host(q_dev[r:r + 1]), host(k_dev[lo:r + 1]), host(v_dev[lo:r + 1]), [r - lo],
                   out[i:i + 1], lse[i:i + 1], f"{what} row {r}")


# ---------------------------------------------------------------------------

def test_small_workload_prefill_then_decode():
    struct = synth.small_structure()
    scale = struct.extra["scale"]
    shape = ha.HeadShape(4, 1, 64, 128, softmax_scale=scale)
    n_pre, steps = int(struct.new[0]), struct.extra["decode_steps"]
    total = n_pre + steps
    for li, kind in enumerate(struct.kinds):
        k = synth.normal_f32((total, 1, 64), "small", li, synth.K_VALUES, DEV)
        v = synth.normal_f32((total, 1, 64), "small", li, synth.V_VALUES, DEV)
        q = synth.normal_f32((total, 4, 64), "small", li, synth.Q_VALUES, DEV)
        for chunks in ([0, n_pre], [0, 128, 256, 384, n_pre]):
            grp_ = grp.HybridGroup(shape, i32(struct.ring_id), struct.num_rings, i32(struct.page_table),
                                   struct.num_pages, kinds=(kind,), fill=float("nan"))
            layer = grp_.layers[0]
            outs, lses = [], []
            for lo, hi in zip(chunks[:-1], chunks[1:]):
                o, l = ha.hybrid_attn_prefill(shape, layer.view, i32([lo]), i32([0, hi - lo]), q[lo:hi], k[lo:hi],
                                              v[lo:hi], max_new=hi - lo)
                append_rows(shape, layer, [lo], k[lo:hi], v[lo:hi], [hi - lo])
                outs.append(o)
                lses.append(l)
            for t in range(n_pre, total):
                append_rows(shape, layer, [t], k[t:t + 1], v[t:t + 1], [1])
                o, l = ha.hybrid_attn_decode(shape, layer.view, i32([t + 1]), q[t:t + 1], t + 1)
                outs.append(o)
                lses.append(l)
            torch.cuda.synchronize()
            # float32 inputs are rounded to bf16 by the library; the oracle sees the same rounding
            kb, vb, qb = (host(x.to(torch.bfloat16)) for x in (k, v, q))
            got_o, got_l = host(torch.cat(outs)), host(torch.cat(lses))
            check_rows(shape, kind, qb, kb, vb, np.arange(total), got_o, got_l, f"small {kind} chunks={chunks}",
                       scale)
            # Against the workload's own float32 inputs (before that rounding): information on what the
            # rounding of Q/K/V to bf16 adds, reported and held to a loose bound only.
            ref_o, ref_l = attend(host(q), host(k), host(v), np.arange(total), kind, shape.window, scale)
            err_o, err_l = float(np.abs(got_o - ref_o).max()), float(np.abs(got_l - ref_l).max())
            print(f"[fp32 inputs] small {kind} chunks={chunks}: max|O - oracle(unrounded fp32)| {err_o:.3e}, "
                  f"max|LSE - oracle| {err_l:.3e}", flush=True)
            assert err_o <= 2e-2 and err_l <= 1e-2


def test_decode_workload_one_step_all_rows():
    struct = synth.decode_structure()
    shape = head_shape(struct)
    b, hist = struct.batch, int(struct.hist[0])
    hq, hkv, d, w = shape.num_q_heads, shape.num_kv_heads, shape.head_dim, shape.window
    group = make_group(struct, shape)
    data = []
    for li, layer in enumerate(group.layers):
        lo = hist - (w - 1) if layer.kind == "swa" else 0          # the history a decode row can see
        n_hist = hist - lo
        k = synth.normal_bf16((b, n_hist + 1, hkv, d), "decode", li, synth.K_VALUES, DEV)
        v = synth.normal_bf16((b, n_hist + 1, hkv, d), "decode", li, synth.V_VALUES, DEV)
        q = synth.normal_bf16((b, hq, d), "decode", li, synth.Q_VALUES, DEV)
        append_rows(shape, layer, [lo] * b, k[:, :n_hist].reshape(-1, hkv, d), v[:, :n_hist].reshape(-1, hkv, d),
                    [n_hist] * b)
        data.append((k, v, q, lo))
    out = [torch.empty(b, hq, d, device=DEV) for _ in group.layers]
    lse = [torch.empty(b, hq, device=DEV) for _ in group.layers]
    plan = grp.plan_decode(group, [x[2] for x in data], [x[0][:, -1].contiguous() for x in data],
                           [x[1][:, -1].contiguous() for x in data], i32([hist] * b), i32([hist + 1] * b),
                           hist + 1, out, lse)
    plan.run()
    torch.cuda.synchronize()
    for li, layer in enumerate(group.layers):
        k, v, q, lo = data[li]
        for s in range(b):
            # positions shifted by lo: the SWA window is translation-invariant
            check_rows(shape, layer.kind, host(q[s:s + 1]), host(k[s]), host(v[s]), [hist - lo],
                       host(out[li][s:s + 1]), host(lse[li][s:s + 1]), f"decode layer {li} seq {s}")


def _chunk_rows(total, chunk, w, rng, extra=24):
    rows = {0, 1, w - 2, w - 1, w, w + 1, total - 1}
    for c0 in range(0, total, chunk):
        rows |= {c0 - 1, c0, c0 + 1, c0 + w - 1, c0 + w}
    rows |= set(rng.integers(0, total, size=extra).tolist())
    return np.array(sorted(r for r in rows if 0 <= r < total))


def test_chunked_workload_sampled_rows():
    struct = synth.chunked_structure()
    shape = head_shape(struct)
    b, total, chunk = struct.batch, int(struct.new[0]), struct.extra["chunk"]
    hq, hkv, d, w = shape.num_q_heads, shape.num_kv_heads, shape.head_dim, shape.window
    group = make_group(struct, shape)
    nch = total // chunk
    vals = [seq_values("chunked", li, b * total, hkv, hq, d) for li in range(len(group.layers))]
    vals = [tuple(x.view(b, total, *x.shape[1:]) for x in kvq) for kvq in vals]
    outs = [torch.empty(b, total, hq, d, device=DEV) for _ in group.layers]
    lses = [torch.empty(b, total, hq, device=DEV) for _ in group.layers]
    cu = i32(np.arange(b + 1) * chunk)
    for c in range(nch):
        sl = slice(c * chunk, (c + 1) * chunk)
        part = lambda x: x[:, sl].reshape(b * chunk, *x.shape[2:]).contiguous()
        o_c = [torch.empty(b * chunk, hq, d, device=DEV) for _ in group.layers]
        l_c = [torch.empty(b * chunk, hq, device=DEV) for _ in group.layers]
        plan = grp.plan_prefill(group, [part(x[2]) for x in vals], [part(x[0]) for x in vals],
                                [part(x[1]) for x in vals], i32([c * chunk] * b), cu, chunk, o_c, l_c)
        plan.run()
        for li in range(len(group.layers)):
            outs[li][:, sl] = o_c[li].view(b, chunk, hq, d)
            lses[li][:, sl] = l_c[li].view(b, chunk, hq)
    torch.cuda.synchronize()
    rng = np.random.default_rng(33)
    for li, layer in enumerate(group.layers):
        for s in range(b):
            rows = _chunk_rows(total, chunk, w, rng)
            rt = torch.as_tensor(rows, device=DEV)
            k, v, q = (x[s] for x in vals[li])
            check_rows_dev(shape, layer.kind, q, k, v, rows, host(outs[li][s][rt]), host(lses[li][s][rt]),
                           f"chunked layer {li} seq {s}")


def test_reuse_workload_window_safe_and_false_hit():
    struct = synth.reuse_structure()
    shape = head_shape(struct)
    w = shape.window
    hq, hkv, d = shape.num_q_heads, shape.num_kv_heads, shape.head_dim
    b = struct.batch
    prefix, suffix = struct.hist.astype(np.int64), struct.new.astype(np.int64)
    reuse_len = np.zeros(b, np.int64)
    for s in range(b):
        req, cached, valid = synth.reuse_tokens(struct, s)
        got = ha.window_safe_match(req, cached, valid, w)
        assert got == window_safe_length(req, cached, valid, w)      # bit-exact length
        reuse_len[s] = got
    n_new = prefix + suffix - reuse_len                 # recomputed tail + new suffix
    group = make_group(struct, shape, fill=float("nan"))
    rng = np.random.default_rng(44)
    check_seqs = set(rng.choice(b, size=6, replace=False).tolist())
    for li, layer in enumerate(group.layers):
        # logical values of positions [first, P+S) per sequence, first = what this layer can need
        first = np.maximum(reuse_len - w, 0) if layer.kind == "swa" else np.zeros(b, np.int64)
        lens = (prefix + suffix - first).astype(np.int64)
        k = synth.normal_bf16((int(lens.sum()), hkv, d), "reuse", li, synth.K_VALUES, DEV)
        v = synth.normal_bf16((int(lens.sum()), hkv, d), "reuse", li, synth.V_VALUES, DEV)
        qc = synth.normal_bf16((int(n_new.sum()), hq, d), "reuse", li, synth.Q_VALUES, DEV)
        offs = np.concatenate([[0], np.cumsum(lens)])
        seq = lambda x, s: x[offs[s]:offs[s + 1]]
        # the reused prefix [first, L) is restored into the pool (ring or pages)
        hist_counts = (reuse_len - first).tolist()
        append_rows(shape, layer, first.tolist(), torch.cat([seq(k, s)[:hist_counts[s]] for s in range(b)]),
                    torch.cat([seq(v, s)[:hist_counts[s]] for s in range(b)]), hist_counts)
        chunk = lambda x: torch.cat([seq(x, s)[hist_counts[s]:] for s in range(b)]).contiguous()
        kc, vc = chunk(k), chunk(v)
        out, lse = ha.hybrid_attn_prefill(shape, layer.view, i32(reuse_len), i32(cu_from_counts(n_new)), qc, kc, vc,
                                          max_new=int(n_new.max()))
        torch.cuda.synchronize()
        cu = cu_from_counts(n_new)
        for s in range(b):
            if layer.kind == "full" and s not in check_seqs:
                continue
            L, T = int(reuse_len[s]), int(prefix[s] - reuse_len[s])
            rel = np.array(sorted({0, 1, T - 1, T, w - 1, w, int(n_new[s]) - 1}
                                  | set(rng.integers(0, int(n_new[s]), size=6).tolist())))
            rel = rel[(rel >= 0) & (rel < n_new[s])]
            # query rows of sequence s, laid out at their positions relative to `first`
            q_s = torch.zeros(int(lens[s]), hq, d, dtype=qc.dtype, device=DEV)
            q_s[hist_counts[s]:] = qc[cu[s]:cu[s + 1]]
            rt = torch.as_tensor(rel, device=DEV)
            check_rows_dev(shape, layer.kind, q_s, seq(k, s), seq(v, s), rel + hist_counts[s],
                           host(out[cu[s]:cu[s + 1]][rt]), host(lse[cu[s]:cu[s + 1]][rt]), f"reuse layer {li} seq {s}")

    # False hit: trust the token match (m = P) instead of the window-safe L.
    # The SWA slots of evicted positions hold invalid data (NaN here), so the
    # restored ring poisons the rows that see them.
    s = int(np.argmax([len(e) for e in struct.extra["evicted"]]))
    assert len(struct.extra["evicted"][s]) > 0
    P, S = int(prefix[s]), int(suffix[s])
    one = ha.HeadShape(hq, hkv, d, w)
    ring = ha.SwaRingPool(one, 1, DEV, fill=float("nan"))
    view = ring.view(i32([0]))
    k, v, q = seq_values("reuse", 0, w + S, hkv, hq, d)         # positions [P-W, P+S)
    k_cache, v_cache = k[:w].clone(), v[:w].clone()
    ev = torch.as_tensor(struct.extra["evicted"][s] - (P - w), device=DEV)
    k_cache[ev] = float("nan")
    v_cache[ev] = float("nan")
    ha.swa_ring_append(one, view, i32([P - w]), i32([0, w]), k_cache, v_cache)
    out, lse = ha.hybrid_attn_prefill(one, view, i32([P]), i32([0, S]), q[w:].contiguous(), k[w:].contiguous(),
                                      v[w:].contiguous(), max_new=S)
    torch.cuda.synchronize()
    # Row i (position P+i) sees positions >= P+i-W+1, so exactly the rows
    # i <= max(evicted) - P + W - 1 read an evicted slot: their scores, and
    # hence their LSE, are corrupted. (The outputs of every row sharing a
    # 64-key tile with such a slot are corrupted too: V is contracted for all
    # rows of a tile at once and 0 * NaN is NaN.)
    e_max = int(struct.extra["evicted"][s].max())
    expect_bad = np.arange(S) <= e_max - P + w - 1
    bad_lse = torch.isnan(lse).any(dim=1).cpu().numpy()
    np.testing.assert_array_equal(bad_lse, expect_bad)
    bad_out = torch.isnan(out).any(dim=(1, 2)).cpu().numpy()
    assert bad_out[expect_bad].all() and not bad_out[w:].any()


def test_ragged_long_decode_split_k():
    struct = synth.ragged_structure()
    shape = head_shape(struct)
    b = struct.batch
    hq, hkv, d, w = shape.num_q_heads, shape.num_kv_heads, shape.head_dim, shape.window
    hist = struct.hist.astype(np.int64)
    group = make_group(struct, shape)
    data = []
    for li, layer in enumerate(group.layers):
        lo = np.maximum(hist - (w - 1), 0) if layer.kind == "swa" else np.zeros(b, np.int64)
        counts = hist - lo
        k = synth.normal_bf16((int(counts.sum()) + b, hkv, d), "ragged", li, synth.K_VALUES, DEV)
        v = synth.normal_bf16((int(counts.sum()) + b, hkv, d), "ragged", li, synth.V_VALUES, DEV)
        q = synth.normal_bf16((b, hq, d), "ragged", li, synth.Q_VALUES, DEV)
        offs = np.concatenate([[0], np.cumsum(counts + 1)])
        hist_rows = torch.cat([k[offs[s]:offs[s + 1] - 1] for s in range(b)])
        hist_vrows = torch.cat([v[offs[s]:offs[s + 1] - 1] for s in range(b)])
        append_rows(shape, layer, lo.tolist(), hist_rows, hist_vrows, counts.tolist())
        new_k = torch.stack([k[offs[s + 1] - 1] for s in range(b)])
        new_v = torch.stack([v[offs[s + 1] - 1] for s in range(b)])
        data.append((k, v, q, new_k, new_v, offs, lo))
    out = [torch.empty(b, hq, d, device=DEV) for _ in group.layers]
    lse = [torch.empty(b, hq, device=DEV) for _ in group.layers]
    max_len = int(hist.max()) + 1
    plan = grp.plan_decode(group, [x[2] for x in data], [x[3] for x in data], [x[4] for x in data],
                           i32(hist), i32(hist + 1), max_len, out, lse)
    plan.run()
    torch.cuda.synchronize()
    assert ha.hybrid_attn_decode_splits(shape, ha.HA_FULL, b, max_len) > 1
    order = np.argsort(hist)
    sample_full = sorted({int(order[0]), int(order[11]), int(order[12]), int(order[19]), int(order[20]),
                          int(order[-1])})
    for li, layer in enumerate(group.layers):
        k, v, q, _, _, offs, lo = data[li]
        seqs = range(b) if layer.kind == "swa" else sample_full
        for s in seqs:
            ks = k[offs[s]:offs[s + 1]].float().cpu().numpy()
            vs_ = v[offs[s]:offs[s + 1]].float().cpu().numpy()
            check_rows(shape, layer.kind, host(q[s:s + 1]), ks, vs_, [int(hist[s] - lo[s])],
                       host(out[li][s:s + 1]), host(lse[li][s:s + 1]), f"ragged layer {li} seq {s} len {hist[s]}")
            del ks, vs_


def test_verify_workload_all_rows():
    """The decode workload's shapes with 4 new tokens per sequence per layer,
    verified by hybrid_attn_verify in the bench's launch configuration
    (automatic split-K for the full layer); every row against the oracle."""
    struct = synth.decode_structure()
    shape = head_shape(struct)
    b, hist, nq = struct.batch, int(struct.hist[0]), 4
    hq, hkv, d, w = shape.num_q_heads, shape.num_kv_heads, shape.head_dim, shape.window
    group = make_group(struct, shape)
    results = []
    for li, layer in enumerate(group.layers):
        lo = hist - (w - 1) if layer.kind == "swa" else 0          # the history the first new token can see
        n_hist = hist - lo
        k = synth.normal_bf16((b, n_hist + nq, hkv, d), "decode", li, synth.K_VALUES + 11, DEV)
        v = synth.normal_bf16((b, n_hist + nq, hkv, d), "decode", li, synth.V_VALUES + 11, DEV)
        q = synth.normal_bf16((b, nq, hq, d), "decode", li, synth.Q_VALUES + 11, DEV)
        append_rows(shape, layer, [lo] * b, k[:, :n_hist].reshape(-1, hkv, d), v[:, :n_hist].reshape(-1, hkv, d),
                    [n_hist] * b)
        out, lse = ha.hybrid_attn_verify(shape, layer.view, i32([hist + nq] * b), q, k[:, n_hist:].contiguous(),
                                         v[:, n_hist:].contiguous(), hist + nq)
        results.append((k, v, q, lo, out, lse))
    torch.cuda.synchronize()
    for li, layer in enumerate(group.layers):
        k, v, q, lo, out, lse = results[li]
        for s in range(b):
            # positions shifted by lo: the SWA window is translation-invariant
            check_rows(shape, layer.kind, host(q[s]), host(k[s]), host(v[s]), np.arange(nq) + (hist - lo),
                       host(out[s]), host(lse[s]), f"verify layer {li} seq {s}")
