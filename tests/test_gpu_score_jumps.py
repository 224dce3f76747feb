"""Decode and verify with scores that jump far above everything seen before.

The decode and verify kernels keep an exp2 reference per query column and
raise it (rescaling O and l) only when a block's scores pass it by a margin;
the INT8 decode path and verify raise it lazily. Keys scaled up at early,
middle and late positions force those raises deep into a row (also across
split-K boundaries), and scaled-up queries widen every row's score range.
The bf16 decode kernel references each block's own maximum, so a row's
dominant key gets probability exactly 1 and its rounding costs nothing; the
lazily raised references of INT8 decode and verify leave the dominant weight
rounded (relative 2^-8), which these rows keep well inside the same bounds
as every other parity test: max |O - oracle| <= 1e-2, max |LSE - oracle| <=
1e-3. Each case prints the error it reaches."""

import numpy as np
import pytest
import torch

import hybrid_sliding_window_gqa_amd as ha
from gpu_util import DEV, LSE_TOL, OUT_TOL, append_history, host, i32, make_generator, oracle_rows, randn_bf16
from oracle.quant import dequantize_rows, quantize_rows
from oracle.attention import attend

pytestmark = pytest.mark.gpu

LENS = [20, 129, 700, 2049]


def spike(k_seq, n):
    for pos in sorted({3, n // 2, n - 20, n - 2}):
        if 0 <= pos < n:
            k_seq[pos] = (k_seq[pos].float() * 40.0).to(torch.bfloat16)


def pools(shape, kind, lens, kv_dtype="bf16", seed=3):
    b = len(lens)
    if kind == ha.HA_SWA:
        pool = ha.SwaRingPool(shape, b + 1, DEV, fill=float("nan"), kv_dtype=kv_dtype)
        return pool.view(i32(list(range(b))[::-1]))
    per = [-(-max(n, 1) // 16) for n in lens]
    perm = np.random.default_rng(seed).permutation(sum(per) + 3)
    table = np.full((b, max(per)), -1, np.int32)
    off = 0
    for s, c in enumerate(per):
        table[s, :c] = perm[off:off + c]
        off += c
    pool = ha.FullPagePool(shape, len(perm), DEV, fill=float("nan"), kv_dtype=kv_dtype)
    return pool.view(i32(table))


def check_rows(out, lse, ref_o, ref_l, v_max, what):
    tol_o = OUT_TOL
    assert np.isfinite(out).all() and np.isfinite(lse).all(), what
    err_o = float(np.abs(out - ref_o).max())
    err_l = float(np.abs(lse - ref_l).max())
    print(f"[score-jump error] {what}: max|O - oracle| {err_o:.3e} (max|V| {v_max:.2f}), "
          f"max|LSE - oracle| {err_l:.3e}", flush=True)
    assert err_o <= tol_o, f"max |O - oracle| = {err_o:.3e} > {tol_o:.3e} {what}"
    assert err_l <= LSE_TOL, f"max |LSE - oracle| = {err_l:.3e} {what}"


def dequantized(x_seq):
    codes, scale = quantize_rows(host(x_seq).astype(np.float64))
    return np.stack([dequantize_rows(codes[:, g], scale[:, g]) for g in range(codes.shape[1])], axis=1)


@pytest.mark.parametrize("kind", [ha.HA_SWA, ha.HA_FULL])
@pytest.mark.parametrize("kv_dtype,splits", [("bf16", 0), ("bf16", 5), ("int8", 0), ("int8", 3)])
def test_decode_with_late_score_jumps(kind, kv_dtype, splits):
    shape = ha.HeadShape(64, 8, 128)
    gen = make_generator(17 + splits)
    hkv, d = shape.num_kv_heads, shape.head_dim
    k = [randn_bf16(gen, n, hkv, d) for n in LENS]
    v = [randn_bf16(gen, n, hkv, d) for n in LENS]
    q = randn_bf16(gen, len(LENS), shape.num_q_heads, d)
    for s, n in enumerate(LENS):
        spike(k[s], n)
    view = pools(shape, kind, LENS, kv_dtype)
    kname = "swa" if kind == ha.HA_SWA else "full"
    starts = [max(0, n - shape.window) if kind == ha.HA_SWA else 0 for n in LENS]
    append_history(shape, view, list(zip(k, v)), starts, LENS)
    for qscale in (1.0, 6.0):
        qq = (q.float() * qscale).to(torch.bfloat16)
        out, lse = ha.hybrid_attn_decode(shape, view, i32(LENS), qq, max(LENS), num_splits=splits)
        torch.cuda.synchronize()
        for s, n in enumerate(LENS):
            if kv_dtype == "int8":
                kd, vd = dequantized(k[s][:n]), dequantized(v[s][:n])
                ref_o, ref_l = attend(host(qq[s])[None], kd, vd, np.array([n - 1]), kname, shape.window)
                v_max = float(np.abs(vd).max())
            else:
                ref_o, ref_l = oracle_rows(host(qq[s:s + 1]), host(k[s]), host(v[s]), [n - 1], kname,
                                           shape.window)
                v_max = float(np.abs(host(v[s])).max())
            check_rows(host(out[s:s + 1]), host(lse[s:s + 1]), ref_o, ref_l, v_max,
                       f"kind={kname} kv={kv_dtype} splits={splits} len={n} qscale={qscale}")


@pytest.mark.parametrize("kind", [ha.HA_SWA, ha.HA_FULL])
@pytest.mark.parametrize("nq,splits,kv_dtype", [(4, 0, "bf16"), (2, 4, "bf16"), (4, 0, "int8"), (2, 4, "int8")])
def test_verify_with_late_score_jumps(kind, nq, splits, kv_dtype):
    shape = ha.HeadShape(64, 8, 128)
    gen = make_generator(29 + nq)
    hq, hkv, d = shape.num_q_heads, shape.num_kv_heads, shape.head_dim
    k = [randn_bf16(gen, n, hkv, d) for n in LENS]
    v = [randn_bf16(gen, n, hkv, d) for n in LENS]
    q = [randn_bf16(gen, n, hq, d) for n in LENS]
    for s, n in enumerate(LENS):
        spike(k[s], n)
        q[s] = (q[s].float() * 6.0).to(torch.bfloat16)
    view = pools(shape, kind, LENS, kv_dtype)
    hist = [n - nq for n in LENS]
    append_history(shape, view, list(zip(k, v)), [0] * len(LENS), hist)
    rows = lambda xs: torch.stack([x[h:h + nq] for x, h in zip(xs, hist)]).contiguous()
    out, lse = ha.hybrid_attn_verify(shape, view, i32(LENS), rows(q), rows(k), rows(v), max(LENS),
                                     num_splits=splits)
    torch.cuda.synchronize()
    kname = "swa" if kind == ha.HA_SWA else "full"
    for s, n in enumerate(LENS):
        pos = np.arange(n - nq, n)
        if kv_dtype == "int8":
            kd, vd = dequantized(k[s][:n]), dequantized(v[s][:n])
            ref_o, ref_l = attend(host(q[s][n - nq:n]), kd, vd, pos, kname, shape.window)
        else:
            ref_o, ref_l = oracle_rows(host(q[s][n - nq:n]), host(k[s]), host(v[s]), pos, kname, shape.window)
        check_rows(host(out[s]), host(lse[s]), ref_o, ref_l, float(np.abs(host(v[s])).max()),
                   f"kind={kname} kv={kv_dtype} nq={nq} splits={splits} len={n}")
