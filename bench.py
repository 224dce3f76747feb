#!/usr/bin/env python3
"""Benchmark of the hybrid SWA/full attention hot path on one MI355X.

Default run (prints ONE JSON line on stdout):
  step     one decode step of a 6:1 layer group (6 SWA layers on W=128 ring
           pools + 1 full layer on a 16-token paged pool) for 64 sequences with
           8192 cached tokens each, Hq/Hkv/D = 64/8/128, bf16 K/V ~ N(0,1):
           per layer, one call appends the new token and attends
           (--separate-append: an append call, then the decode call).
  value    decode HBM GB/s = algorithmic bytes per step / step time, where
           algorithmic bytes = K/V rows the queries see + Q read + O (fp32)
           and LSE written.
  prefill  chunked causal prefill of 4 x 32768 tokens in 8192-token chunks
           through the same group (attend, then append): TFLOP/s with
           4*D flops per visible (query head, key) pair.
  roofline achieved/peak of the dominant kernel (the full-layer decode
           call), timed with HIP events on the launch stream.
  verify, int8_kv, ragged, reuse
           the decode pools with 4 new tokens per sequence; the decode step
           and that verify step on INT8 pools; ragged long-context decode (24
           sequences, 1K to 1M cached tokens, split-K); prefix-reuse prefill
           (32 sequences, window-safe reuse) -- each skippable with
           --no-<name>.
  cpu_baseline  the fp64 oracle on a bounded sample of the decode step.

Inputs are synthetic and resident in HBM before timing starts. Options select
other workloads (--workload reuse|ragged) for extra JSON lines.
"""

from __future__ import annotations

import argparse
import ctypes
import hashlib
import json
import os
import sys
import time

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, published
MFMA_BF16_PEAK_TFLOPS = 2500.0  # MI355X dense bf16 matrix, published
METRIC = "decode attn HBM GB/s (% peak) + prefill TFLOP/s (% MFMA peak), SWA:full 6:1"


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def parse():
    p = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=50)
    p.add_argument("--warmup", type=int, default=10)
    p.add_argument("--restore-groups", type=int, default=4,
                   help="groups in the stack the restore workload pipelines (its pools are per group)")
    p.add_argument("--workload", choices=["decode", "reuse", "ragged", "chunked", "copy", "verify", "restore",
                                          "decode_int8", "verify_int8"],
                   default="decode",
                   help="copy: 2 GiB elementwise copy, the known-size kernel that scales HBM counters")
    p.add_argument("--prefill-passes", type=int, default=3)
    p.add_argument("--no-prefill", action="store_true", help="skip the chunked-prefill part")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--no-verify", action="store_true", help="skip the multi-token verify part")
    p.add_argument("--no-int8", action="store_true", help="skip the INT8-pool decode part")
    p.add_argument("--no-ragged", action="store_true", help="skip the ragged long-context decode part")
    p.add_argument("--no-reuse", action="store_true", help="skip the prefix-reuse prefill part")
    p.add_argument("--cpu-seconds", type=float, default=15.0, help="target oracle time for the CPU sample")
    p.add_argument("--cpu-prefill-seconds", type=float, default=10.0,
                   help="target oracle time for the prefill CPU sample")
    p.add_argument("--eager", action="store_true", help="launch calls directly instead of replaying a HIP graph")
    p.add_argument("--cold-bytes", type=float, default=768e6,
                   help="rotate decode steps over ring copies so that a ring is read again only after this "
                        "many bytes of other rings (0: one copy)")
    p.add_argument("--no-ceilings", action="store_true", help="skip the copy / read-pattern / MFMA ceilings")
    p.add_argument("--no-restore", action="store_true", help="skip the layer-wise restore part")
    p.add_argument("--no-quant-error", action="store_true", help="skip the INT8 quantization-error sample")
    p.add_argument("--cpu-ragged-seconds", type=float, default=8.0)
    p.add_argument("--cpu-reuse-seconds", type=float, default=8.0)
    p.add_argument("--separate-append", action="store_true",
                   help="decode step as append call + decode call per layer instead of one fused call")
    return p.parse_args()


# ---------------------------------------------------------------------------
# algorithmic work (closed forms of the visibility rule)

def visible_keys(t, kind, window):
    t = np.asarray(t, dtype=np.int64)
    return np.minimum(t + 1, window) if kind == "swa" else t + 1


def visible_pairs_range(hist, n, kind, window):
    """Sum over query positions hist..hist+n-1 of the visible key count."""
    t = np.arange(hist, hist + n, dtype=np.int64)
    return int(visible_keys(t, kind, window).sum())


def kv_bytes_per_token(shape):
    return shape.num_kv_heads * shape.head_dim * 2 * 2      # K and V, bf16


def decode_layer_bytes(shape, kind, kv_len):
    keys = visible_keys(np.asarray(kv_len) - 1, kind, shape.window).sum()
    b = len(kv_len)
    q = b * shape.num_q_heads * shape.head_dim * 2
    o = b * shape.num_q_heads * shape.head_dim * 4
    l = b * shape.num_q_heads * 4
    return int(keys) * kv_bytes_per_token(shape) + q + o + l


# ---------------------------------------------------------------------------
# HBM traffic per dispatch, from the committed rocprofv3 counter summaries

def sources_digest(paths):
    """sha256 over the given repository files, in order (identifies the kernel
    build that a counter summary was taken from)."""
    h = hashlib.sha256()
    for rel in paths:
        with open(os.path.join(HERE, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def profile_traffic(name):
    """Calibrated HBM bytes per dispatch recorded in profiles/<name>, or None
    when the summary is missing or the kernel's sources changed since the
    counters were taken."""
    try:
        with open(os.path.join(HERE, "profiles", name), encoding="utf-8") as f:
            lines = f.read().splitlines()
    except OSError:
        return None
    fields = {}
    for line in lines:
        key, sep, val = line.partition(":")
        if sep and key.strip() in ("traffic_bytes_per_dispatch", "sources", "sources_sha256"):
            fields[key.strip()] = val.strip()
    try:
        if sources_digest(fields["sources"].split()) != fields["sources_sha256"]:
            return None
        return int(float(fields["traffic_bytes_per_dispatch"]))
    except (KeyError, ValueError, OSError):
        return None


DECODE_PROFILE = "decode_kernel_full_decode64x8192_pmc.txt"
PREFILL_PROFILE = "prefill_kernel_full_chunked4x32768_pmc.txt"
VERIFY_PROFILE = "verify_kernel_full_verify64x8192_pmc.txt"
RAGGED_PROFILE = "decode_kernel_full_ragged24_pmc.txt"
REUSE_PROFILE = "prefill_kernel_full_reuse32_pmc.txt"
SWA_DECODE_PROFILE = "decode_kernel_swa_decode64x8192_pmc.txt"
SWA_PREFILL_PROFILE = "prefill_kernel_swa_chunked4x32768_pmc.txt"


def run_copy(torch, args, device):
    """Known-size plain copy (dst = -src over 2 GiB of bf16) used to scale
    the FETCH_SIZE / WRITE_SIZE counters to bytes."""
    n = 1 << 30
    src = torch.empty(n, dtype=torch.bfloat16, device=device).fill_(1.0)
    dst = torch.empty_like(src)
    torch.neg(src, out=dst)
    torch.cuda.synchronize()
    reps = 3
    t0 = time.perf_counter()
    for _ in range(reps):
        torch.neg(src, out=dst)
    torch.cuda.synchronize()
    dt = (time.perf_counter() - t0) / reps
    # write-only stream of the same size (a fill)
    dst.fill_(0.5)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(reps):
        dst.fill_(0.5)
    torch.cuda.synchronize()
    dw = (time.perf_counter() - t0) / reps
    # read-only stream of the same buffer (a max-reduction), for the achievable read rate
    torch.amax(src)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(reps):
        torch.amax(src)
    torch.cuda.synchronize()
    dr = (time.perf_counter() - t0) / reps
    return {"workload": "calibration copy: dst = -src, 2 GiB bf16 each way", "bytes_read": 2 * n,
            "bytes_written": 2 * n, "ms": dt * 1e3, "copy_gbs": 4 * n / dt / 1e9,
            "read_only_gbs": 2 * n / dr / 1e9, "write_only_gbs": 2 * n / dw / 1e9}


def timed_events(torch, n):
    return [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(n)]


def build_decode(torch, ha, grp, synth, struct, device, workload, fuse=True, kv_dtype="bf16", share=None):
    """Pools filled with each sequence's history; per-layer new-token tensors.

    share: an earlier build of the same structure. The new copy then uses
    that build's full-layer pool and its Q/K/V/O tensors and owns only its
    SWA rings (filled with the same values), so a step can rotate over ring
    copies whose total exceeds the last-level cache while the full layer
    keeps reading one 16-token-paged pool."""
    shape = ha.HeadShape(struct.shape.num_q_heads, struct.shape.num_kv_heads, struct.shape.head_dim,
                         struct.shape.window)
    b = struct.batch
    hist = struct.hist.astype(np.int64)
    ring_id = torch.as_tensor(struct.ring_id, device=device)
    table = torch.as_tensor(struct.page_table, device=device)
    pools = {}
    if share is not None:
        sgroup = share[1]
        pools = {li: layer.pool for li, layer in enumerate(sgroup.layers) if layer.kind == "full"}
    group = grp.HybridGroup(shape, ring_id, struct.num_rings, table, struct.num_pages, kv_dtype=kv_dtype,
                            pools=pools)
    hkv, hq, d, w = shape.num_kv_heads, shape.num_q_heads, shape.head_dim, shape.window
    logical = []   # per layer: (k_hist, v_hist, first_position) host-side recipe for the oracle
    q_l, k_l, v_l, out_l, lse_l = [], [], [], [], []
    for li, layer in enumerate(group.layers):
        if share is not None and li in pools:
            continue
        if layer.kind == "swa":
            start = np.maximum(hist - (w - 1), 0)
        else:
            start = np.zeros(b, np.int64)
        counts = (hist - start).astype(np.int64)
        total = int(counts.sum())
        k_hist = synth.normal_bf16((total, hkv, d), workload, li, synth.K_VALUES, device)
        v_hist = synth.normal_bf16((total, hkv, d), workload, li, synth.V_VALUES, device)
        cu = torch.as_tensor(np.concatenate([[0], np.cumsum(counts)]).astype(np.int32), device=device)
        pos0 = torch.as_tensor(start.astype(np.int32), device=device)
        fn = ha.swa_ring_append if layer.kind == "swa" else ha.full_pool_append
        fn(shape, layer.view, pos0, cu, k_hist, v_hist)
        if share is None:
            logical.append((k_hist, v_hist, start, cu.cpu().numpy()))
            q_l.append(synth.normal_bf16((b, hq, d), workload, li, synth.Q_VALUES, device))
            k_l.append(synth.normal_bf16((b, hkv, d), workload, li, synth.K_VALUES + 3, device))
            v_l.append(synth.normal_bf16((b, hkv, d), workload, li, synth.V_VALUES + 3, device))
            out_l.append(torch.empty(b, hq, d, dtype=torch.float32, device=device))
            lse_l.append(torch.empty(b, hq, dtype=torch.float32, device=device))
        del k_hist, v_hist
    if share is not None:
        data = share[3]
        q_l, k_l, v_l, out_l, lse_l = data["q"], data["k"], data["v"], data["out"], data["lse"]
    else:
        data = dict(q=q_l, k=k_l, v=v_l, out=out_l, lse=lse_l, logical=logical, hist=hist)
    # SWA pool size is O(W) per sequence and layer, independent of the history length
    swa_layers = sum(1 for layer in group.layers if layer.kind == "swa")
    tok = kv8_bytes_per_token(shape) if kv_dtype == "int8" else kv_bytes_per_token(shape)
    assert group.pool_bytes()["swa"] == swa_layers * struct.num_rings * w * tok, "SWA pool is not O(W)"
    pos = torch.as_tensor(hist.astype(np.int32), device=device)
    kv_len = torch.as_tensor((hist + 1).astype(np.int32), device=device)
    plan = grp.plan_decode(group, q_l, k_l, v_l, pos, kv_len, int(hist.max()) + 1, out_l, lse_l,
                           fuse_append=fuse)
    torch.cuda.synchronize()
    return shape, group, plan, data


_CAPTURE_STREAM = None


def capture_stream(torch):
    """The one side stream every graph capture of this run uses. A process
    gets few hardware queues (4 by default) and streams share them round-robin
    in creation order, so a stream per capture would leave later streams (the
    restore's copy stream) on the same queue as the compute stream, where
    they serialize instead of overlapping."""
    global _CAPTURE_STREAM
    if _CAPTURE_STREAM is None:
        _CAPTURE_STREAM = torch.cuda.Stream()
    return _CAPTURE_STREAM


def rotation_copies(args, ring_bytes):
    """Ring copies so that a ring is read again only after at least
    args.cold_bytes of other rings (0: one copy, warm replay only)."""
    if args.cold_bytes <= 0 or ring_bytes <= 0:
        return 1
    return max(2, 1 + -(-int(args.cold_bytes) // int(ring_bytes)))


def time_steps(torch, plans, args, labels_of_interest=None):
    """Times one step (a plan per pool copy) four ways, all with inputs
    resident in HBM:
      cold   graph replays rotating over the copies, so every ring is read
             after more than the last-level cache of other rings (the
             headline; K steps bracketed by synchronize, wall clock);
      steps  the same rotation with HIP events around each replay (median,
             p10, p90 of the per-step times);
      warm   graph replays of copy 0 only (its rings stay cache-resident);
      eager  the rotation launched call by call, no graph.
    And the per-call durations (HIP events on the launch stream, eager
    launches rotating over the copies)."""
    stream = torch.cuda.current_stream()
    graphs = []
    if not args.eager:
        side = capture_stream(torch)
        for pl in plans:
            pl.run()                                # eager warm call before capture
            torch.cuda.synchronize()
            side.wait_stream(stream)
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g, stream=side):
                pl.run()
            graphs.append(g)
        torch.cuda.synchronize()
    n = len(plans)

    def step(i):
        if graphs:
            graphs[i % n].replay()
        else:
            plans[i % n].run()

    def wall(fn, k):
        for i in range(args.warmup):
            fn(i)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for i in range(k):
            fn(i)
        torch.cuda.synchronize()
        return (time.perf_counter() - t0) / k

    cold = wall(step, args.steps)
    warm = wall(lambda i: graphs[0].replay() if graphs else plans[0].run(), args.steps)
    eager = wall(lambda i: plans[i % n].run(), args.steps)
    evs = timed_events(torch, args.steps)
    for i in range(args.warmup):
        step(i)
    for i, (e0, e1) in enumerate(evs):
        e0.record(stream)
        step(i)
        e1.record(stream)
    torch.cuda.synchronize()
    per_step = np.array([e0.elapsed_time(e1) for e0, e1 in evs])
    ncalls = len(plans[0].calls)
    cevs = timed_events(torch, ncalls)
    sums = np.zeros(ncalls)
    reps = max(5, min(args.steps, 20))
    for r in range(reps):
        plans[r % n].run_timed(cevs, stream)
        torch.cuda.synchronize()
        sums += np.array([a.elapsed_time(c) for a, c in cevs])
    return {
        "cold_s": cold, "warm_s": warm, "eager_s": eager,
        "step_ms_p10": float(np.percentile(per_step, 10)), "step_ms_p50": float(np.median(per_step)),
        "step_ms_p90": float(np.percentile(per_step, 90)), "copies": n,
        "call_ms": sums / reps, "labels": list(plans[0].labels),
    }


def build_copies(torch, ha, grp, synth, struct, args, device, fuse=True, kv_dtype="bf16"):
    """Copy 0 of the decode pools, then ring copies sharing its full pool."""
    first = build_decode(torch, ha, grp, synth, struct, device, struct.workload, fuse=fuse, kv_dtype=kv_dtype)
    ring_bytes = first[1].pool_bytes()["swa"]
    copies = [first]
    for _ in range(rotation_copies(args, ring_bytes) - 1):
        copies.append(build_decode(torch, ha, grp, synth, struct, device, struct.workload, fuse=fuse,
                                   kv_dtype=kv_dtype, share=first))
    return copies, ring_bytes


def timing_fields(t, step_bytes):
    """JSON fields of time_steps() for a step of step_bytes algorithmic bytes."""
    return {
        "cold_ms_per_step": round(t["cold_s"] * 1e3, 4),
        "step_ms_p10": round(t["step_ms_p10"], 4), "step_ms_p50": round(t["step_ms_p50"], 4),
        "step_ms_p90": round(t["step_ms_p90"], 4),
        "warm_ms_per_step": round(t["warm_s"] * 1e3, 4),
        "warm_gbs": round(step_bytes / t["warm_s"] / 1e9, 2),
        "eager_ms_per_step": round(t["eager_s"] * 1e3, 4),
        "eager_gbs": round(step_bytes / t["eager_s"] / 1e9, 2),
        "ring_copies_rotated": t["copies"],
    }


def run_decode(torch, ha, grp, synth, struct, args, device):
    copies, ring_bytes = build_copies(torch, ha, grp, synth, struct, args, device, fuse=not args.separate_append)
    shape, group, plan, data = copies[0]
    kv_len = data["hist"] + 1
    # per layer: the attention's bytes plus the new token's K/V read and written
    # by the append (fused into the decode call, or a call of its own)
    layer_append = struct.batch * kv_bytes_per_token(shape) * 2
    per_layer_bytes = [decode_layer_bytes(shape, layer.kind, kv_len) + layer_append for layer in group.layers]
    step_bytes = sum(per_layer_bytes)
    append_bytes = len(group.layers) * layer_append
    t = time_steps(torch, [c[2] for c in copies], args)
    call_ms = t["call_ms"]
    labels = t["labels"]
    by_label = dict(zip(labels, call_ms.tolist()))
    full_idx = [i for i, lab in enumerate(labels) if lab.startswith("decode") and "full" in lab]
    swa_idx = [i for i, lab in enumerate(labels) if lab.startswith("decode") and "swa" in lab]
    app_idx = [i for i, lab in enumerate(labels) if lab.startswith("append")]
    full_ms = float(np.mean(call_ms[full_idx]))
    swa_ms = float(np.mean(call_ms[swa_idx]))
    full_layer = [i for i, layer in enumerate(group.layers) if layer.kind == "full"][0]
    swa_layer = [i for i, layer in enumerate(group.layers) if layer.kind == "swa"][0]
    call_extra = 0 if app_idx else layer_append     # the decode call appends only when fused
    full_bytes = per_layer_bytes[full_layer] - layer_append + call_extra
    swa_bytes = per_layer_bytes[swa_layer] - layer_append + call_extra
    pool = group.pool_bytes()
    full_used = int(kv_len.sum()) * kv_bytes_per_token(shape)
    info = {
        "step_bytes": step_bytes,
        "append_bytes": append_bytes,
        **timing_fields(t, step_bytes),
        "full_decode_ms": full_ms,
        "full_decode_gbs": full_bytes / full_ms / 1e6,
        "swa_decode_ms": swa_ms,
        "swa_decode_gbs": swa_bytes / swa_ms / 1e6,
        "swa_decode_bytes": swa_bytes,
        "append_ms_avg": float(np.mean(call_ms[app_idx])) if app_idx else None,
        "fused_append": not app_idx,
        "calls_ms": by_label,
        "graph": not args.eager,
        "splits_full": ha.hybrid_attn_decode_splits(shape, ha.HA_FULL, struct.batch, int(kv_len.max())),
        "swa_pool_bytes": pool["swa"],
        "swa_pool_bytes_per_ring_layer": pool["swa"] // (struct.num_rings * 6),
        "kv_bytes_vs_all_full": round((pool["swa"] // struct.num_rings * struct.batch + full_used)
                                      / (len(group.layers) * full_used), 4),
    }
    return shape, group, data, t["cold_s"], step_bytes, full_bytes, info, copies


def kv8_bytes_per_token(shape):
    """INT8 pools: codes of K and V plus one float32 scale each, per kv head."""
    return shape.num_kv_heads * (shape.head_dim * 2 + 8)


def run_decode_int8(torch, ha, grp, synth, args, device):
    """The decode workload on INT8 pools: per layer one call that quantizes
    and appends the new token and attends (--separate-append: an append call
    and a decode call), timed like the bf16 step; and the full-layer call."""
    struct = synth.decode_structure()
    copies, _ = build_copies(torch, ha, grp, synth, struct, args, device, fuse=not args.separate_append,
                             kv_dtype="int8")
    shape, group, plan, data = copies[0]
    b = struct.batch
    kv_len = data["hist"] + 1
    hq, d = shape.num_q_heads, shape.head_dim
    qol = b * hq * (d * 2 + d * 4 + 4)                       # Q read, O and LSE written
    append = b * (shape.num_kv_heads * shape.head_dim * 2 * 2 + kv8_bytes_per_token(shape))
    per_layer = [int(visible_keys(kv_len - 1, layer.kind, shape.window).sum()) * kv8_bytes_per_token(shape) + qol
                 for layer in group.layers]
    step_bytes = sum(per_layer) + append * len(group.layers)
    t = time_steps(torch, [c[2] for c in copies], args)
    dt = t["cold_s"]
    call_ms = t["call_ms"]
    lab = t["labels"]
    full_ms = float(np.mean([call_ms[i] for i, x in enumerate(lab) if x.startswith("decode") and "full" in x]))
    swa_ms = float(np.mean([call_ms[i] for i, x in enumerate(lab) if x.startswith("decode") and "swa" in x]))
    app = [call_ms[i] for i, x in enumerate(lab) if x.startswith("append")]
    app_ms = float(np.mean(app)) if app else 0.0
    full_layer = [i for i, layer in enumerate(group.layers) if layer.kind == "full"][0]
    full_bytes = per_layer[full_layer] + (0 if app else append)    # a fused call also appends
    value = step_bytes / dt / 1e9
    log(f"[bench] int8 decode step {dt * 1e3:.3f} ms, {value:.1f} GB/s, {b / dt:.0f} tokens/s; full call "
        f"{full_ms * 1e3:.1f} us ({full_bytes / full_ms / 1e6:.0f} GB/s), swa call {swa_ms * 1e3:.1f} us, "
        f"append {app_ms * 1e3:.1f} us")
    return {
        "metric": "decode attn HBM GB/s (% peak) on INT8 KV pools, SWA:full 6:1",
        "value": round(value, 2),
        "unit": "GB/s",
        "ms_per_step": round(dt * 1e3, 4),
        "tokens_per_s": round(b / dt, 1),
        "pct_peak_hbm": round(100.0 * value / HBM_PEAK_GBS, 2),
        "step_bytes": step_bytes,
        **timing_fields(t, step_bytes),
        "workload": (f"decode: {b} sequences x {int(kv_len[0]) - 1} cached tokens on INT8 pools (per-token "
                     f"scales), one 6:1 group, per layer "
                     + ("an append call then a decode call" if app else "one call (quantize, append, attend)")),
        "full_call_us": round(full_ms * 1e3, 2),
        "full_call_gbs": round(full_bytes / full_ms / 1e6, 2),
        "full_call_frac": round(full_bytes / full_ms / 1e6 / HBM_PEAK_GBS, 4),
        "full_call_bytes": full_bytes,
        "swa_call_us": round(swa_ms * 1e3, 2),
        "append_call_us": round(app_ms * 1e3, 2),
        "calls_ms": dict(zip(lab, call_ms.tolist())),
        "copies": copies,
    }


def int8_quant_error(torch, synth, q8, args):
    """max |O_int8 - O_ref| and |LSE_int8 - LSE_ref| on sampled sequences of
    the INT8 decode step. O_ref is plain float32 attention (torch products
    and softmax on the GPU) over the unquantized bf16 K/V the pools were
    quantized from: the output change that the 8-bit format causes."""
    shape, group, _plan, data = q8["copies"][0]
    hist = data["hist"]
    hq, hkv, d = shape.num_q_heads, shape.num_kv_heads, shape.head_dim
    g = hq // hkv
    scale = shape.softmax_scale if shape.softmax_scale > 0 else 1.0 / float(np.sqrt(d))
    rows = [0, len(hist) // 3, 2 * len(hist) // 3, len(hist) - 1]
    err_o = err_l = 0.0
    for li, layer in enumerate(group.layers):
        if li not in (0, len(group.layers) - 1):
            continue
        k_hist, v_hist, start, cu = data["logical"][li]
        for b in rows:
            k = torch.cat([k_hist[cu[b]:cu[b + 1]], data["k"][li][b:b + 1]]).float()
            v = torch.cat([v_hist[cu[b]:cu[b + 1]], data["v"][li][b:b + 1]]).float()
            if layer.kind == "swa":                  # keys at positions > t - W
                k, v = k[-shape.window:], v[-shape.window:]
            q = data["q"][li][b].float().reshape(hkv, g, d)
            s = torch.bmm(q, k.permute(1, 2, 0).contiguous()) * scale          # [hkv, g, n]
            lse = torch.logsumexp(s, dim=-1)
            o = torch.bmm(torch.softmax(s, dim=-1), v.permute(1, 0, 2).contiguous())
            err_o = max(err_o, float((data["out"][li][b] - o.reshape(hq, d)).abs().max()))
            err_l = max(err_l, float((data["lse"][li][b] - lse.reshape(hq)).abs().max()))
    return {"max_abs_o": err_o, "max_abs_lse": err_l,
            "sample": f"sequences {rows} of the INT8 decode step, SWA layer 0 and the full layer, all query "
                      f"heads, against float32 attention over the unquantized bf16 K/V ({int(hist[0]) + 1} keys)"}


def verify_layer_bytes(shape, kind, t0, nq, kv8=False):
    """Algorithmic bytes of one multi-token verify call: the history keys the
    queries need (all t0 for full layers; the W-1 before t0 for SWA layers),
    the new tokens' K/V read (bf16) and appended (in the pool's format), Q
    read, O (fp32) and LSE written."""
    t0 = np.asarray(t0, dtype=np.int64)
    hist = t0 if kind == "full" else np.minimum(t0, shape.window - 1)
    b = len(t0)
    tok = kv_bytes_per_token(shape)
    pool_tok = kv8_bytes_per_token(shape) if kv8 else tok
    q = b * nq * shape.num_q_heads * shape.head_dim * 2
    o = b * nq * shape.num_q_heads * shape.head_dim * 4
    l = b * nq * shape.num_q_heads * 4
    return int(hist.sum()) * pool_tok + b * nq * (tok + pool_tok) + q + o + l


def run_verify(torch, ha, grp, synth, args, device, nq=4, kv_dtype="bf16"):
    """The decode workload's pools (bf16, or INT8 with kv_dtype="int8"), one
    step verifying nq tokens per sequence in every layer of the group, timed
    like the decode step (cold rotation over ring copies, warm, eager); and
    the full-layer call alone."""
    kv8 = kv_dtype == "int8"
    struct = synth.decode_structure()
    copies, _ = build_copies(torch, ha, grp, synth, struct, args, device, kv_dtype=kv_dtype)
    shape, group, _plan, data = copies[0]
    b = struct.batch
    hist = data["hist"].astype(np.int64)
    hq, hkv, d = shape.num_q_heads, shape.num_kv_heads, shape.head_dim
    kv_len = torch.as_tensor((hist + nq).astype(np.int32), device=device)
    max_len = int(hist.max()) + nq
    q_l, k_l, v_l, out_l, lse_l = [], [], [], [], []
    for li in range(len(group.layers)):
        q_l.append(synth.normal_bf16((b, nq, hq, d), struct.workload, li, synth.Q_VALUES + 11, device))
        k_l.append(synth.normal_bf16((b, nq, hkv, d), struct.workload, li, synth.K_VALUES + 11, device))
        v_l.append(synth.normal_bf16((b, nq, hkv, d), struct.workload, li, synth.V_VALUES + 11, device))
        out_l.append(torch.empty(b, nq, hq, d, dtype=torch.float32, device=device))
        lse_l.append(torch.empty(b, nq, hq, dtype=torch.float32, device=device))
    plans = [grp.plan_verify(c[1], q_l, k_l, v_l, kv_len, max_len, out_l, lse_l) for c in copies]
    t = time_steps(torch, plans, args)
    dt = t["cold_s"]
    full_i = [i for i, layer in enumerate(group.layers) if layer.kind == "full"][0]
    full_ms = float(t["call_ms"][full_i])
    step_bytes = sum(verify_layer_bytes(shape, layer.kind, hist, nq, kv8) for layer in group.layers)
    full_bytes = verify_layer_bytes(shape, "full", hist, nq, kv8)
    value = step_bytes / dt / 1e9
    log(f"[bench] verify step ({kv_dtype} pools) {dt * 1e3:.3f} ms, {value:.1f} GB/s, "
        f"{b * nq / dt:.0f} tokens verified/s; full call {full_ms * 1e3:.1f} us ({full_bytes / full_ms / 1e6:.0f} GB/s)")
    return {
        "metric": ("multi-token verify decode attn HBM GB/s (% peak), SWA:full 6:1"
                   + (", INT8 KV pools" if kv8 else "")),
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(dt * 1e3, 4),
        "higher_is_better": True,
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": (f"verify: {b} sequences x {int(hist[0])} cached tokens + {nq} new tokens each "
                                f"(causal among them), one 6:1 group, Hq/Hkv/D {hq}/{hkv}/{d}"
                                + (", INT8 pools (per-token scales)" if kv8 else "")),
                   "global_batch": b, "tokens_per_sequence": nq, "parallelism": "none (1 GPU)"},
        "pct_peak_hbm": round(100.0 * value / HBM_PEAK_GBS, 2),
        "tokens_verified_per_s": round(b * nq / dt, 1),
        **timing_fields(t, step_bytes),
        "roofline": {"bound": "hbm", "achieved": round(full_bytes / full_ms / 1e6, 2), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(full_bytes / full_ms / 1e6 / HBM_PEAK_GBS, 4),
                     "traffic": None if kv8 else profile_traffic(VERIFY_PROFILE),
                     "kernel": (f"hybrid_attn_verify, full layer (verify_kernel<128,full,bf16,2,{kv_dtype}> "
                                "+ reduce)"),
                     "bytes_per_launch": full_bytes},
    }


def prefill_pass_flops(shape, kinds, batch, total, chunk):
    """Algorithmic flops of one chunked prefill pass through the group."""
    flops = {"swa": 0, "full": 0}
    for c in range(total // chunk):
        for kind in set(kinds):
            pairs = visible_pairs_range(c * chunk, chunk, kind, shape.window) * batch * shape.num_q_heads
            flops[kind] += pairs * 4 * shape.head_dim * kinds.count(kind)
    return flops


def run_chunked(torch, ha, grp, synth, args, device, cpu_seconds=0.0):
    struct = synth.chunked_structure()
    shape = ha.HeadShape(struct.shape.num_q_heads, struct.shape.num_kv_heads, struct.shape.head_dim,
                         struct.shape.window)
    b, total, chunk = struct.batch, int(struct.new[0]), struct.extra["chunk"]
    nchunks = total // chunk
    hq, hkv, d = shape.num_q_heads, shape.num_kv_heads, shape.head_dim
    group = grp.HybridGroup(shape, torch.as_tensor(struct.ring_id, device=device), struct.num_rings,
                            torch.as_tensor(struct.page_table, device=device), struct.num_pages)
    t_chunk = b * chunk
    # per layer, per chunk: rows of the chunk for all sequences, contiguous
    qs, ks, vs = [], [], []
    for li in range(len(group.layers)):
        q = synth.normal_bf16((nchunks, t_chunk, hq, d), "chunked", li, synth.Q_VALUES, device)
        k = synth.normal_bf16((nchunks, t_chunk, hkv, d), "chunked", li, synth.K_VALUES, device)
        v = synth.normal_bf16((nchunks, t_chunk, hkv, d), "chunked", li, synth.V_VALUES, device)
        qs.append(q)
        ks.append(k)
        vs.append(v)
    outs = [torch.empty(t_chunk, hq, d, dtype=torch.float32, device=device) for _ in group.layers]
    lses = [torch.empty(t_chunk, hq, dtype=torch.float32, device=device) for _ in group.layers]
    cu = torch.as_tensor(np.arange(b + 1, dtype=np.int32) * chunk, device=device)
    plans = []
    for c in range(nchunks):
        hist = torch.full((b,), c * chunk, dtype=torch.int32, device=device)
        plans.append(grp.plan_prefill(group, [q[c] for q in qs], [k[c] for k in ks], [v[c] for v in vs],
                                      hist, cu, chunk, outs, lses))
    flops = prefill_pass_flops(shape, list(group.kinds), b, total, chunk)
    total_flops = flops["swa"] + flops["full"]

    def one_pass():
        for pl in plans:
            pl.run()

    one_pass()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.prefill_passes):
        one_pass()
    torch.cuda.synchronize()
    dt = (time.perf_counter() - t0) / args.prefill_passes

    stream = torch.cuda.current_stream()
    call_ms = {}
    for pl in plans:
        evs = timed_events(torch, len(pl.calls))
        pl.run_timed(evs, stream)
        torch.cuda.synchronize()
        for lab, (a, e) in zip(pl.labels, evs):
            call_ms.setdefault(lab, []).append(a.elapsed_time(e))
    full_ms = sum(v for lab, vals in call_ms.items() if lab.startswith("prefill") and "full" in lab for v in vals)
    swa_ms = sum(v for lab, vals in call_ms.items() if lab.startswith("prefill") and "swa" in lab for v in vals)
    n_swa = list(group.kinds).count("swa")
    swa_bytes_per_layer = 0
    for c in range(nchunks):
        rows = t_chunk
        swa_bytes_per_layer += rows * hq * d * 2 + rows * hq * d * 4 + rows * hq * 4 + rows * kv_bytes_per_token(shape)
    res = {
        "workload": f"chunked causal prefill: {b} sequences x {total} tokens in {chunk}-token chunks, "
                    f"one 6:1 group (6 SWA W={shape.window} + 1 full), Hq/Hkv/D {hq}/{hkv}/{d}, bf16",
        "pass_ms": dt * 1e3,
        "tflops": total_flops / dt / 1e12,
        "pct_mfma_peak": 100.0 * total_flops / dt / 1e12 / MFMA_BF16_PEAK_TFLOPS,
        "flops_per_pass": total_flops,
        "full_layer_ms": full_ms,
        "full_layer_tflops": flops["full"] / (full_ms * 1e-3) / 1e12,
        "swa_layers_ms": swa_ms,
        "swa_layer_gbs": swa_bytes_per_layer * n_swa / (swa_ms * 1e-3) / 1e9,
        "swa_call_bytes": swa_bytes_per_layer // nchunks,
        "swa_call_traffic": profile_traffic(SWA_PREFILL_PROFILE),
        "roofline": {
            "bound": "mfma",
            "achieved": flops["full"] / (full_ms * 1e-3) / 1e12,
            "peak": MFMA_BF16_PEAK_TFLOPS,
            "unit": "TFLOP/s",
            "frac": flops["full"] / (full_ms * 1e-3) / 1e12 / MFMA_BF16_PEAK_TFLOPS,
            "traffic": profile_traffic(PREFILL_PROFILE),
            "kernel": "hybrid_attn_prefill, full layer (stage_chunk_kernel + prefill_kernel<128,full> + prefill_merge_kernel), "
                      f"mean over the {nchunks} chunk calls",
            "flops_per_launch": flops["full"] / nchunks,
        },
    }
    if cpu_seconds > 0:
        log("[bench] cpu baseline (oracle), prefill rows")
        res["cpu_baseline"] = cpu_baseline_prefill(torch, shape, group, qs, ks, vs, chunk, cpu_seconds)
        res["cpu_baseline"]["extrapolated_pass_s"] = total_flops / (res["cpu_baseline"]["value"] * 1e12)
        res["cpu_baseline"]["extrapolated"] = True
    del qs, ks, vs, outs, lses, group
    torch.cuda.empty_cache()
    return res


def blas_thread_count():
    try:
        import threadpoolctl
        return max((i.get("num_threads", 1) for i in threadpoolctl.threadpool_info()), default=1)
    except Exception:  # pragma: no cover
        return 1


def run_reuse(torch, ha, grp, synth, args, device, cpu_seconds=0.0):
    """Prefix-reuse prefill: per sequence, the window-safe match L of the
    request against its cached prefix, the reused history restored (pages
    [0, L); ring positions [L-W, L)), then one pass of the recomputed tail +
    new suffix (n = P + S - L tokens at [L, L+n)) through the 6:1 group
    (attend, then append)."""
    struct = synth.reuse_structure()
    shape = ha.HeadShape(struct.shape.num_q_heads, struct.shape.num_kv_heads, struct.shape.head_dim,
                         struct.shape.window)
    b, w = struct.batch, shape.window
    hq, hkv, d = shape.num_q_heads, shape.num_kv_heads, shape.head_dim
    prefix, suffix = struct.hist.astype(np.int64), struct.new.astype(np.int64)
    reuse_len = np.array([ha.window_safe_match(*synth.reuse_tokens(struct, s), w) for s in range(b)], np.int64)
    n_new = prefix + suffix - reuse_len
    group = grp.HybridGroup(shape, torch.as_tensor(struct.ring_id, device=device), struct.num_rings,
                            torch.as_tensor(struct.page_table, device=device), struct.num_pages)
    log(f"[bench] reuse: restoring history ({int(reuse_len.sum())} cached positions)")
    # sequence 0's logical K/V of one SWA and the full layer, kept for the oracle baseline
    oracle_layers = {"swa": list(group.kinds).index("swa"), "full": list(group.kinds).index("full")}
    seq0_hist = {}
    for li, layer in enumerate(group.layers):
        first = np.maximum(reuse_len - w, 0) if layer.kind == "swa" else np.zeros(b, np.int64)
        counts = reuse_len - first
        total = int(counts.sum())
        if total == 0:
            continue
        k = synth.normal_bf16((total, hkv, d), "reuse", li, synth.K_VALUES, device)
        v = synth.normal_bf16((total, hkv, d), "reuse", li, synth.V_VALUES, device)
        fn = ha.swa_ring_append if layer.kind == "swa" else ha.full_pool_append
        fn(shape, layer.view, torch.as_tensor(first.astype(np.int32), device=device),
           torch.as_tensor(np.concatenate([[0], np.cumsum(counts)]).astype(np.int32), device=device), k, v)
        if cpu_seconds > 0 and oracle_layers.get(layer.kind) == li:
            c0 = int(counts[0])
            seq0_hist[layer.kind] = (k[:c0].float().cpu().numpy(), v[:c0].float().cpu().numpy(), int(first[0]))
        del k, v
    t_new = int(n_new.sum())
    qs, ks, vs, outs, lses = [], [], [], [], []
    for li in range(len(group.layers)):
        qs.append(synth.normal_bf16((t_new, hq, d), "reuse", li, synth.Q_VALUES + 3, device))
        ks.append(synth.normal_bf16((t_new, hkv, d), "reuse", li, synth.K_VALUES + 3, device))
        vs.append(synth.normal_bf16((t_new, hkv, d), "reuse", li, synth.V_VALUES + 3, device))
        outs.append(torch.empty(t_new, hq, d, dtype=torch.float32, device=device))
        lses.append(torch.empty(t_new, hq, dtype=torch.float32, device=device))
    hist = torch.as_tensor(reuse_len.astype(np.int32), device=device)
    cu = torch.as_tensor(np.concatenate([[0], np.cumsum(n_new)]).astype(np.int32), device=device)
    plan = grp.plan_prefill(group, qs, ks, vs, hist, cu, int(n_new.max()), outs, lses)
    flops = {"swa": 0, "full": 0}
    for kind in ("swa", "full"):
        pairs = sum(visible_pairs_range(int(reuse_len[s]), int(n_new[s]), kind, w) for s in range(b))
        flops[kind] = pairs * hq * 4 * d * list(group.kinds).count(kind)
    total_flops = flops["swa"] + flops["full"]
    torch.cuda.synchronize()
    plan.run()                      # warm (re-running appends rewrites the same rows)
    torch.cuda.synchronize()
    passes = max(1, args.prefill_passes)
    t0 = time.perf_counter()
    for _ in range(passes):
        plan.run()
    torch.cuda.synchronize()
    dt = (time.perf_counter() - t0) / passes
    evs = timed_events(torch, len(plan.calls))
    plan.run_timed(evs, torch.cuda.current_stream())
    torch.cuda.synchronize()
    call_ms = dict(zip(plan.labels, [a.elapsed_time(e) for a, e in evs]))
    full_ms = sum(v for lab, v in call_ms.items() if lab.startswith("prefill") and "full" in lab)
    full_tf = flops["full"] / (full_ms * 1e-3) / 1e12
    cpu = None
    if cpu_seconds > 0 and len(seq0_hist) == 2:
        log("[bench] cpu baseline (oracle), prefix-reuse rows")
        n0 = int(n_new[0])
        seq0 = {"L": int(reuse_len[0]), "n": n0}
        for kind, li in oracle_layers.items():
            kh, vh, first0 = seq0_hist[kind]
            seq0[kind] = (qs[li][:n0].float().cpu().numpy(),
                          np.concatenate([kh, ks[li][:n0].float().cpu().numpy()]),
                          np.concatenate([vh, vs[li][:n0].float().cpu().numpy()]), first0)
        cpu = cpu_baseline_reuse(torch, shape, list(group.kinds), seq0, cpu_seconds, total_flops)
    return {
        "metric": METRIC,
        "workload": f"prefix-reuse prefill: {b} sequences, cached prefix P~U[4096,65536] with evicted SWA slots, "
                    f"window-safe reuse L (total {int(reuse_len.sum())}), recomputed tail + suffix U[512,2048] "
                    f"= {t_new} new tokens, one 6:1 group, Hq/Hkv/D {hq}/{hkv}/{d}, bf16",
        "pass_ms": dt * 1e3,
        "tflops": total_flops / dt / 1e12,
        "pct_mfma_peak": 100.0 * total_flops / dt / 1e12 / MFMA_BF16_PEAK_TFLOPS,
        "flops_per_pass": total_flops,
        "full_layer_ms": full_ms,
        "full_layer_tflops": full_tf,
        "roofline": {"bound": "mfma", "achieved": full_tf, "peak": MFMA_BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                     "frac": full_tf / MFMA_BF16_PEAK_TFLOPS, "traffic": profile_traffic(REUSE_PROFILE),
                     "kernel": "hybrid_attn_prefill, full layer (stage_chunk_kernel + prefill_kernel<128,full> + prefill_merge_kernel)",
                     "flops_per_launch": flops["full"]},
        "full_call_compulsory_bytes": int(t_new * hq * d * (2 + 4) + t_new * hq * 4
                                          + (t_new + int(reuse_len.sum())) * kv_bytes_per_token(shape)),
        "mean_recomputed_tail": float((prefix - reuse_len).mean()),
        "data": "synthetic",
        **({"cpu_baseline": cpu} if cpu else {}),
    }


def run_restore(torch, ha, grp, synth, args, device):
    """The prefix-reuse workload with its reused history held in pinned host
    memory, over a stack of groups: each layer's rows are copied to the
    device and scattered into its pool on a copy stream, layer l's restore
    overlapping earlier layers' prefill. Times the restores alone, the
    prefill passes alone and the overlapped pipeline, and the best that
    pipeline can do given per-layer times (copy l must end before compute l
    starts)."""
    struct = synth.reuse_structure()
    shape = ha.HeadShape(struct.shape.num_q_heads, struct.shape.num_kv_heads, struct.shape.head_dim,
                         struct.shape.window)
    b, w = struct.batch, shape.window
    hq, hkv, d = shape.num_q_heads, shape.num_kv_heads, shape.head_dim
    ng = args.restore_groups
    prefix, suffix = struct.hist.astype(np.int64), struct.new.astype(np.int64)
    reuse_len = np.array([ha.window_safe_match(*synth.reuse_tokens(struct, s), w) for s in range(b)], np.int64)
    n_new = prefix + suffix - reuse_len
    ring_id = torch.as_tensor(struct.ring_id, device=device)
    table = torch.as_tensor(struct.page_table, device=device)
    groups = [grp.HybridGroup(shape, ring_id, struct.num_rings, table, struct.num_pages) for _ in range(ng)]
    nl = len(groups[0].layers)
    log(f"[bench] restore: {ng} groups, pinning {int(reuse_len.sum())} cached positions per full layer")
    first, counts, k_rows, v_rows = [], [], [], []
    for li, layer in enumerate(groups[0].layers):
        f = np.maximum(reuse_len - w, 0) if layer.kind == "swa" else np.zeros(b, np.int64)
        c = reuse_len - f
        first.append(f.tolist())
        counts.append(c.tolist())
        k_rows.append(synth.normal_bf16((int(c.sum()), hkv, d), "reuse", li, synth.K_VALUES, device))
        v_rows.append(synth.normal_bf16((int(c.sum()), hkv, d), "reuse", li, synth.V_VALUES, device))
    # every group restores the same pinned rows (a bandwidth workload): one
    # pinned copy, one set of staging buffers on the one copy stream
    host_kv = grp.HostKv(groups[0], first, counts, k_rows, v_rows)
    del k_rows, v_rows
    restores = [grp.RestorePlan(groups[0], host_kv)]
    restores += [grp.RestorePlan(g, host_kv, staging_from=restores[0]) for g in groups[1:]]
    t_new = int(n_new.sum())
    qs, ks, vs, outs, lses = [], [], [], [], []
    for li in range(nl):
        qs.append(synth.normal_bf16((t_new, hq, d), "reuse", li, synth.Q_VALUES + 3, device))
        ks.append(synth.normal_bf16((t_new, hkv, d), "reuse", li, synth.K_VALUES + 3, device))
        vs.append(synth.normal_bf16((t_new, hkv, d), "reuse", li, synth.V_VALUES + 3, device))
        outs.append(torch.empty(t_new, hq, d, dtype=torch.float32, device=device))
        lses.append(torch.empty(t_new, hq, dtype=torch.float32, device=device))
    hist = torch.as_tensor(reuse_len.astype(np.int32), device=device)
    cu = torch.as_tensor(np.concatenate([[0], np.cumsum(n_new)]).astype(np.int32), device=device)
    # the groups' passes share their inputs and outputs (in order on one stream)
    plans = [grp.plan_prefill(g, qs, ks, vs, hist, cu, int(n_new.max()), outs, lses) for g in groups]
    compute, copy_stream = torch.cuda.current_stream(), torch.cuda.Stream()
    reps = max(2, args.prefill_passes)

    def timed(fn):
        fn()                                    # warm
        torch.cuda.synchronize()
        ts = []
        for _ in range(reps):
            t0 = time.perf_counter()
            fn()
            torch.cuda.synchronize()
            ts.append(time.perf_counter() - t0)
        return float(np.median(ts))

    def restore_all():
        for r in restores:
            r.run(copy_stream)

    def prefill_all():
        for p in plans:
            p.run(compute)

    t_restore = timed(restore_all)
    t_compute = timed(prefill_all)
    t_overlap = timed(lambda: grp.run_restore_overlapped(restores, plans, compute, copy_stream))
    # per-layer times of group 0, each stream alone
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(nl)]
    for li in range(nl):
        ev[li][0].record(copy_stream)
        restores[0].run_layer(li, copy_stream)
        ev[li][1].record(copy_stream)
    torch.cuda.synchronize()
    r_ms = [e0.elapsed_time(e1) for e0, e1 in ev]
    by_layer = grp.layer_calls(plans[0], nl)
    ptr = ctypes.c_void_p(compute.cuda_stream)
    for li in range(nl):
        ev[li][0].record(compute)
        for call in by_layer[li]:
            call(ptr)
        ev[li][1].record(compute)
    torch.cuda.synchronize()
    p_ms = [e0.elapsed_time(e1) for e0, e1 in ev]
    copy_end = comp_end = 0.0
    for _ in range(ng):
        for li in range(nl):
            copy_end += r_ms[li]
            comp_end = max(comp_end, copy_end) + p_ms[li]
    nbytes = host_kv.nbytes() * ng
    hidden = t_restore + t_compute - t_overlap
    frac = hidden / min(t_restore, t_compute)
    log(f"[bench] restore {t_restore * 1e3:.2f} ms ({nbytes / t_restore / 1e9:.1f} GB/s host to device), "
        f"prefill {t_compute * 1e3:.2f} ms, overlapped {t_overlap * 1e3:.2f} ms (schedule bound "
        f"{comp_end:.2f} ms); {hidden * 1e3:.2f} ms hidden ({100 * frac:.1f}% of the shorter)")
    log("[bench] per layer restore ms " + " ".join(f"{x:.2f}" for x in r_ms)
        + " | prefill ms " + " ".join(f"{x:.2f}" for x in p_ms))
    return {
        "metric": "layer-wise KV restore from pinned host memory overlapped with prefill",
        "workload": f"prefix-reuse prefill ({b} sequences, window-safe reuse L total {int(reuse_len.sum())}, "
                    f"{t_new} new tokens) over a stack of {ng} 6:1 groups, each layer's reused history "
                    f"restored from pinned host memory (full layer: all L positions; SWA layers: the last W)",
        "groups": ng,
        "restored_bytes": nbytes,
        "restore_ms": t_restore * 1e3,
        "h2d_gbs": nbytes / t_restore / 1e9,
        "prefill_ms": t_compute * 1e3,
        "serial_ms": (t_restore + t_compute) * 1e3,
        "overlapped_ms": t_overlap * 1e3,
        "schedule_bound_ms": comp_end,
        "hidden_ms": hidden * 1e3,
        "overlap_fraction_of_shorter": frac,
        "overlap_fraction_of_allowed": hidden / ((t_restore + t_compute) - comp_end * 1e-3),
        "layer_restore_ms": r_ms,
        "layer_prefill_ms": p_ms,
        "data": "synthetic",
    }


def run_ceilings(torch, shape, group, data, device):
    """Achievable ceilings measured in the same run, next to the published
    peaks: a plain 2 GiB copy and a read-only reduction (torch), decode's
    own read pattern over the decode workload's full pool with and without
    the non-temporal bit (include/ha_probe.h), and the matrix cores alone."""
    from hybrid_sliding_window_gqa_amd import _lib

    lib = _lib.load()
    res = run_copy(torch, None, device)
    out = {"copy_gbs": round(res["copy_gbs"], 1), "write_only_gbs": round(res["write_only_gbs"], 1)}
    stream = torch.cuda.current_stream()
    sptr = ctypes.c_void_p(stream.cuda_stream)
    full = [layer for layer in group.layers if layer.kind == "full"][0]
    kv_len_np = (data["hist"] + 1).astype(np.int32)
    kv_len = torch.as_tensor(kv_len_np, device=device)
    b = len(kv_len_np)
    sink = torch.empty(b * shape.num_kv_heads * 256, dtype=torch.int32, device=device)
    nbytes = int(np.sum(-(-kv_len_np // 16))) * shape.num_kv_heads * 16 * shape.head_dim * 2 * 2
    c_shape, c_view = shape.c(), full.view.c()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)

    def timed(launch, reps=10):
        for _ in range(3):
            launch()
        torch.cuda.synchronize()
        e0.record(stream)
        for _ in range(reps):
            launch()
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / reps * 1e-3

    for nt, key in ((1, "decode_pattern_read_nt_gbs"), (0, "decode_pattern_read_gbs")):
        dt = timed(lambda: _lib.check(lib.ha_probe_paged_read(ctypes.byref(c_shape), ctypes.byref(c_view),
                                                               kv_len.data_ptr(), b, sink.data_ptr(), nt, sptr)))
        out[key] = round(nbytes / dt / 1e9, 1)
    iters = 8192
    fsink = torch.empty(1024 * 256, dtype=torch.float32, device=device)
    best = (0.0, 0)
    for wgs in (256, 512, 1024):             # 1, 2 and 4 waves per SIMD
        dt = timed(lambda: _lib.check(lib.ha_probe_mfma_bf16(wgs, iters, fsink.data_ptr(), sptr)), reps=5)
        best = max(best, (wgs * 4 * iters * 8 * 16384 / dt / 1e12, wgs))
    out["mfma_bf16_tflops"] = round(best[0], 1)
    # Matrix cores beside vector work (two waves per SIMD, one workgroup per CU): how much of one
    # wave's exp2/FMA work hides under another wave's products on the same SIMD.
    csink = torch.empty(256 * 512, dtype=torch.float32, device=device)
    cms = {}
    for mode, name in enumerate(("matrix_only", "split_waves", "in_phase", "ping_pong", "vector_only")):
        dt = timed(lambda m=mode: _lib.check(lib.ha_probe_coissue(m, 256, 2000, csink.data_ptr(), sptr)), reps=3)
        cms[name] = round(dt * 1e3, 3)
    out["coissue_ms"] = cms
    out["what"] = ("copy: dst = -src over 2 GiB; write_only: a fill of 2 GiB; decode_pattern_read: every K/V block of the decode "
                   f"workload's full pool ({nbytes} B) read as the full-layer decode kernel walks it, no "
                   "arithmetic (nt: non-temporal loads, as decode issues them); mfma: v_mfma_f32_16x16x32_bf16 "
                   f"with register operands, best of 1, 2 and 4 waves per SIMD ({best[1] // 256} per SIMD); "
                   "coissue_ms: ha_probe_coissue modes 0-4 (96 MFMAs and 96 exp2/FMA pairs per wave and "
                   "iteration, 2000 iterations, 8 waves per CU): matrix blocks only, waves 0-3 matrix next to "
                   "waves 4-7 vector, both in phase between barriers, ping-pong, vector blocks only")
    del sink, fsink, csink
    return out


def cpu_baseline_reuse(torch, shape, kinds, seq0, target_s, total_flops):
    """The fp64 oracle on seeded rows of sequence 0 of the prefix-reuse pass
    (its reused history plus its new tokens; full and SWA layer alternately,
    all query heads) for about target_s seconds; TFLOP/s of algorithmic
    flops and the whole pass's time extrapolated from that rate."""
    sys.path.insert(0, HERE)
    from oracle.attention import attend

    w, d, hq = shape.window, shape.head_dim, shape.num_q_heads
    reuse_len, n_new = seq0["L"], seq0["n"]
    rng = np.random.default_rng(11)
    done_flops, done_s, rows = 0, 0.0, {"full": 0, "swa": 0}
    step = 0
    while done_s < target_s:
        kind = ("full", "swa")[step % 2]
        step += 1
        q, k, v, first = seq0[kind]            # q [n, Hq, D]; k/v rows from position `first`
        pos = np.sort(rng.choice(n_new, size=min(4, n_new), replace=False)) + reuse_len
        t0 = time.perf_counter()
        attend(q[pos - reuse_len], k, v, pos - first, kind, w)
        done_s += time.perf_counter() - t0
        rows[kind] += len(pos)
        done_flops += int(visible_keys(pos, kind, w).sum()) * hq * 4 * d
    rate = done_flops / done_s
    return {
        "value": rate / 1e12,
        "unit": "TFLOP/s",
        "cores": int(blas_thread_count()),
        "kind": "oracle",
        "sample": f"{rows['full']} full-layer and {rows['swa']} SWA-layer query rows of sequence 0 (reused "
                  f"{reuse_len}, new {n_new}; seeded), all {hq} query heads, {done_s:.1f} s of fp64 NumPy",
        "extrapolated_pass_s": total_flops / rate,
        "extrapolated": True,
    }


def cpu_baseline_prefill(torch, shape, group, qs, ks, vs, chunk, target_s):
    """Time the fp64 oracle on seeded sample rows of the chunked prefill
    (sequence 0; full and SWA layer alternately; all query heads) until about
    target_s seconds of CPU work; report algorithmic TFLOP/s."""
    sys.path.insert(0, HERE)
    from oracle.attention import attend

    w, d, hq = shape.window, shape.head_dim, shape.num_q_heads
    nchunks = qs[0].shape[0]
    total = nchunks * chunk
    rng = np.random.default_rng(7)
    layers = {kind: group.kinds.index(kind) for kind in ("full", "swa")}
    logical = {}
    for kind, li in layers.items():
        k = ks[li][:, :chunk].reshape(total, *ks[li].shape[2:]).float().cpu().numpy()
        v = vs[li][:, :chunk].reshape(total, *vs[li].shape[2:]).float().cpu().numpy()
        logical[kind] = (k, v)
    done_flops, done_s, rows = 0, 0.0, {"full": 0, "swa": 0}
    step = 0
    while done_s < target_s:
        kind = ("full", "swa")[step % 2]
        step += 1
        li = layers[kind]
        pos = np.sort(rng.integers(0, total, size=4))
        q = np.stack([qs[li][p // chunk, p % chunk].float().cpu().numpy() for p in pos])
        k, v = logical[kind]
        t0 = time.perf_counter()
        if kind == "full":
            attend(q, k, v, pos, kind, w)
        else:
            for i, p in enumerate(pos):         # the window's keys only, positions shifted
                lo = max(0, int(p) - w + 1)
                attend(q[i:i + 1], k[lo:p + 1], v[lo:p + 1], [int(p) - lo], kind, w)
        done_s += time.perf_counter() - t0
        rows[kind] += len(pos)
        done_flops += int(visible_keys(pos, kind, w).sum()) * hq * 4 * d
    return {
        "value": done_flops / done_s / 1e12,
        "unit": "TFLOP/s",
        "cores": int(blas_thread_count()),
        "kind": "oracle",
        "sample": f"{rows['full']} full-layer and {rows['swa']} SWA-layer query rows of sequence 0 "
                  f"(seeded positions in [0, {total})), all {hq} query heads, {done_s:.1f} s of fp64 NumPy",
    }


def cpu_baseline(torch, shape, group, data, target_s):
    """Time the fp64 oracle on whole sequences of the decode step (all 7
    layers each) until about target_s seconds of CPU work, and express it in
    the metric's unit (algorithmic bytes per second)."""
    sys.path.insert(0, HERE)
    from oracle.attention import attend

    blas_threads = blas_thread_count()
    w = shape.window
    hist = data["hist"]
    b_total = len(hist)
    done_bytes, done_s, seqs = 0, 0.0, 0
    host = {}
    for b in (i % b_total for i in range(100 * b_total)):   # passes over the step until target_s
        if b not in host:
            # host copies of this sequence's logical K/V (generator tensors, not pools)
            per_layer = []
            for li, layer in enumerate(group.layers):
                k_hist, v_hist, start, cu = data["logical"][li]
                k = torch.cat([k_hist[cu[b]:cu[b + 1]], data["k"][li][b:b + 1]]).float().cpu().numpy()
                v = torch.cat([v_hist[cu[b]:cu[b + 1]], data["v"][li][b:b + 1]]).float().cpu().numpy()
                q = data["q"][li][b:b + 1].float().cpu().numpy()
                per_layer.append((layer.kind, k, v, q, int(hist[b] - start[b])))
            host[b] = per_layer
        per_layer = host[b]
        t0 = time.perf_counter()
        for kind, k, v, q, t in per_layer:
            attend(q, k, v, [t], kind, w)
        done_s += time.perf_counter() - t0
        seqs += 1
        for li, layer in enumerate(group.layers):
            done_bytes += decode_layer_bytes(shape, layer.kind, [hist[b] + 1])
        if done_s >= target_s:
            break
    return {
        "value": done_bytes / done_s / 1e9,
        "unit": "GB/s",
        "cores": int(blas_threads),
        "kind": "oracle",
        "sample": f"{seqs} sequence rows of the decode step ({seqs / b_total:.2f} passes over its {b_total} "
                  f"sequences), all 7 layers, all query heads ({done_s:.1f} s of fp64 NumPy)",
    }


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (got --gpus {args.gpus}); this library has no "
              "multi-GPU path", file=sys.stderr)
        return 2
    import torch

    import hybrid_sliding_window_gqa_amd as ha
    import synth
    from hybrid_sliding_window_gqa_amd import group as grp

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        return 2
    device = torch.device("cuda:0")
    torch.cuda.set_device(device)

    if args.workload == "chunked":
        res = run_chunked(torch, ha, grp, synth, args, device)
        print(json.dumps(res))
        return 0
    if args.workload == "copy":
        print(json.dumps(run_copy(torch, args, device)))
        return 0

    if args.workload == "reuse":
        print(json.dumps(run_reuse(torch, ha, grp, synth, args, device)))
        return 0
    if args.workload in ("verify", "verify_int8"):
        kv_dtype = "int8" if args.workload == "verify_int8" else "bf16"
        print(json.dumps(run_verify(torch, ha, grp, synth, args, device, kv_dtype=kv_dtype)))
        return 0
    if args.workload == "restore":
        print(json.dumps(run_restore(torch, ha, grp, synth, args, device)))
        return 0
    if args.workload == "decode_int8":
        q8 = run_decode_int8(torch, ha, grp, synth, args, device)
        if not args.no_quant_error:
            q8["quant_error"] = int8_quant_error(torch, synth, q8, args)
        del q8["copies"]                # the pools, kept for the quantization-error sample
        print(json.dumps(q8))
        return 0
    struct = {"decode": synth.decode_structure, "ragged": synth.ragged_structure}[args.workload]()
    log(f"[bench] workload={args.workload} building inputs")
    shape, group, data, dt, step_bytes, full_bytes, info, copies = run_decode(torch, ha, grp, synth, struct, args,
                                                                               device)
    value = step_bytes / dt / 1e9
    log(f"[bench] step {dt * 1e3:.3f} ms cold ({value:.1f} GB/s; p10/p50/p90 {info['step_ms_p10']:.3f}/"
        f"{info['step_ms_p50']:.3f}/{info['step_ms_p90']:.3f} ms over {info['ring_copies_rotated']} ring copies), "
        f"warm {info['warm_ms_per_step']:.3f} ms, eager {info['eager_ms_per_step']:.3f} ms; full decode "
        f"{info['full_decode_ms'] * 1e3:.1f} us ({info['full_decode_gbs']:.0f} GB/s), swa decode "
        f"{info['swa_decode_ms'] * 1e3:.1f} us ({info['swa_decode_gbs']:.0f} GB/s)")
    if args.workload == "decode":
        wl = (f"decode: {struct.batch} sequences x {int(struct.hist[0])} cached tokens, one 6:1 group "
              f"(6 SWA layers W={shape.window} ring + 1 full layer, 16-token pages, seeded page permutation), "
              f"Hq/Hkv/D {shape.num_q_heads}/{shape.num_kv_heads}/{shape.head_dim}, 1 new token per sequence")
    else:
        wl = (f"ragged decode: {struct.batch} sequences, cached lengths 12xU[1K,64K] 8xU[64K,256K] "
              f"4xU[256K,1M] (total {int(struct.hist.sum())}), one 6:1 group, split-K over full pages")
    line = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(dt * 1e3, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": wl, "global_batch": struct.batch, "seq_len": int(struct.hist.max()) + 1,
                   "parallelism": "none (1 GPU)"},
        "pct_peak_hbm": round(100.0 * value / HBM_PEAK_GBS, 2),
        "timing": ("value and ms_per_step: graph replays rotating over ring copies (cold caches: each ring "
                   "is read again only after more than the last-level cache of other rings); warm: replays "
                   "of one copy; eager: the rotation launched call by call"),
        "decode_detail": {k: (round(v, 4) if isinstance(v, float) else v) for k, v in info.items()
                          if k != "calls_ms"},
        "roofline": {
            "bound": "hbm",
            "achieved": round(info["full_decode_gbs"], 2),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(info["full_decode_gbs"] / HBM_PEAK_GBS, 4),
            "traffic": profile_traffic(DECODE_PROFILE if args.workload == "decode" else RAGGED_PROFILE),
            "kernel": ("hybrid_attn_decode, full layer (decode_kernel<128,full>"
                       + (f" + decode_reduce_kernel<128>, {info['splits_full']} splits)" if info["splits_full"] > 1
                          else ", one split per sequence: no merge)")),
            "bytes_per_launch": full_bytes,
        },
    }
    if args.workload == "decode":
        line["decode_detail"]["swa_decode_traffic"] = profile_traffic(SWA_DECODE_PROFILE)
    if args.workload == "decode" and not args.no_ceilings:
        log("[bench] ceilings")
        line["ceilings"] = run_ceilings(torch, shape, group, data, device)
        log(f"[bench] ceilings {line['ceilings']}")
    del copies
    if args.workload == "decode" and not args.no_prefill:
        log("[bench] chunked prefill")
        line["prefill"] = run_chunked(torch, ha, grp, synth, args, device,
                                      0.0 if args.no_cpu_baseline else args.cpu_prefill_seconds)
        log(f"[bench] prefill {line['prefill']['tflops']:.1f} TFLOP/s, full layer "
            f"{line['prefill']['full_layer_tflops']:.1f} TFLOP/s")
    if args.workload == "decode" and not args.no_verify:
        log("[bench] multi-token verify")
        v = run_verify(torch, ha, grp, synth, args, device)
        line["verify"] = {k: v[k] for k in ("value", "unit", "ms_per_step", "pct_peak_hbm", "tokens_verified_per_s",
                                            "step_ms_p50", "warm_ms_per_step", "eager_ms_per_step")}
        line["verify"]["workload"] = v["config"]["workload"]
        line["verify"]["full_call_gbs"] = v["roofline"]["achieved"]
        line["verify"]["roofline"] = v["roofline"]
        torch.cuda.empty_cache()
    if args.workload == "decode" and not args.no_int8:
        log("[bench] decode on INT8 pools")
        q8 = run_decode_int8(torch, ha, grp, synth, args, device)
        line["int8_kv"] = {k: q8[k] for k in ("value", "unit", "ms_per_step", "tokens_per_s", "pct_peak_hbm",
                                              "workload", "full_call_us", "full_call_gbs", "full_call_frac",
                                              "swa_call_us", "append_call_us", "step_ms_p50", "warm_ms_per_step",
                                              "eager_ms_per_step")}
        if not args.no_quant_error:
            line["int8_kv"]["quant_error"] = int8_quant_error(torch, synth, q8, args)
        del q8
        torch.cuda.empty_cache()
        log("[bench] multi-token verify on INT8 pools")
        v8 = run_verify(torch, ha, grp, synth, args, device, kv_dtype="int8")
        line["int8_kv"]["verify"] = {k: v8[k] for k in ("value", "unit", "ms_per_step", "pct_peak_hbm",
                                                        "tokens_verified_per_s")}
        line["int8_kv"]["verify"]["full_call_gbs"] = v8["roofline"]["achieved"]
        del v8
        torch.cuda.empty_cache()
    if args.workload == "decode" and not args.no_ragged:
        log("[bench] ragged long-context decode")
        torch.cuda.empty_cache()        # its 17.7 GB of pools come from fresh allocations
        rstruct = synth.ragged_structure()
        _, rgroup, rdata, rdt, rbytes, rfull, rinfo, rcopies = run_decode(torch, ha, grp, synth, rstruct, args,
                                                                          device)
        line["ragged"] = {
            "value": round(rbytes / rdt / 1e9, 2), "unit": "GB/s", "ms_per_step": round(rdt * 1e3, 4),
            "pct_peak_hbm": round(100.0 * rbytes / rdt / 1e9 / HBM_PEAK_GBS, 2),
            "workload": (f"ragged decode: {rstruct.batch} sequences, cached lengths 12xU[1K,64K] 8xU[64K,256K] "
                         f"4xU[256K,1M] (total {int(rstruct.hist.sum())}), one 6:1 group, split-K over full pages"),
            "full_call_gbs": round(rinfo["full_decode_gbs"], 2), "splits_full": rinfo["splits_full"],
            **{k: rinfo[k] for k in ("step_ms_p50", "warm_ms_per_step", "eager_ms_per_step", "ring_copies_rotated")},
            "roofline": {"bound": "hbm", "achieved": round(rinfo["full_decode_gbs"], 2), "peak": HBM_PEAK_GBS,
                         "unit": "GB/s", "frac": round(rinfo["full_decode_gbs"] / HBM_PEAK_GBS, 4),
                         "traffic": profile_traffic(RAGGED_PROFILE),
                         "kernel": f"hybrid_attn_decode, full layer (decode_kernel<128,full> + decode_reduce_kernel"
                                   f"<128>, {rinfo['splits_full']} splits)",
                         "bytes_per_launch": rfull},
        }
        if not args.no_cpu_baseline:
            log("[bench] cpu baseline (oracle), ragged decode")
            cb = cpu_baseline(torch, shape, rgroup, rdata, args.cpu_ragged_seconds)
            cb["extrapolated_step_s"] = rbytes / (cb["value"] * 1e9)
            cb["extrapolated"] = True
            line["ragged"]["cpu_baseline"] = cb
        del rgroup, rdata, rcopies
        torch.cuda.empty_cache()
    if args.workload == "decode" and not args.no_reuse:
        log("[bench] prefix-reuse prefill")
        ru = run_reuse(torch, ha, grp, synth, args, device,
                       0.0 if args.no_cpu_baseline else args.cpu_reuse_seconds)
        line["reuse"] = {k: ru[k] for k in ("workload", "pass_ms", "tflops", "pct_mfma_peak", "full_layer_tflops",
                                            "mean_recomputed_tail", "full_call_compulsory_bytes", "roofline")}
        line["reuse"]["full_layer_frac"] = ru["roofline"]["frac"]
        if "cpu_baseline" in ru:
            line["reuse"]["cpu_baseline"] = ru["cpu_baseline"]
        torch.cuda.empty_cache()
    if args.workload == "decode" and not args.no_restore:
        log("[bench] layer-wise restore")
        rs = run_restore(torch, ha, grp, synth, args, device)
        line["restore"] = {k: rs[k] for k in ("workload", "groups", "restored_bytes", "restore_ms", "h2d_gbs",
                                              "prefill_ms", "serial_ms", "overlapped_ms", "schedule_bound_ms",
                                              "hidden_ms", "overlap_fraction_of_shorter",
                                              "overlap_fraction_of_allowed")}
        torch.cuda.empty_cache()
    if args.workload == "decode":
        line["targets"] = {
            "decode_step_pct_hbm": line["pct_peak_hbm"], "decode_target_pct_hbm": 70.0,
            "decode_met": line["pct_peak_hbm"] >= 70.0,
        }
        if "prefill" in line:
            pf = 100.0 * line["prefill"]["roofline"]["frac"]
            line["targets"].update({"prefill_full_layer_pct_mfma": round(pf, 2),
                                    "prefill_target_pct_mfma": 50.0, "prefill_met": pf >= 50.0})
    if args.workload == "decode" and not args.no_cpu_baseline:
        log("[bench] cpu baseline (oracle)")
        line["cpu_baseline"] = cpu_baseline(torch, shape, group, data, args.cpu_seconds)
        line["cpu_baseline"]["extrapolated_step_s"] = step_bytes / (line["cpu_baseline"]["value"] * 1e9)
    print(json.dumps(line), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
