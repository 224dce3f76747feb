"""a9: one 6:1 hybrid layer group -- six SWA layers (W-slot ring pools) then
one full layer (paged pool) -- and its per-step call order.

The pages describe 70 layers of which 60 use a 128-token sliding window and
10 attend to everything, interleaved 6:1 (htx.com news section 工程一;
blog.hotdry.top 2026-06-09 sections "Hybrid SWA：用 1/7 计算量捕获长程依赖"
and "生产级调参清单"); the last layer of each group of seven is taken as the
full one. Each layer owns its own pool, and the two pool kinds are separate
allocations ("KVCache系统重构：让缓存真正省下来", youleyou.com).

Plans pre-marshal every argument of a step's library calls once, so running a
step is a sequence of ctypes calls with no per-call tensor inspection: cheap
enough to keep the GPU fed, and capturable in a HIP graph because each call
takes the current stream at run time.

Step order:
  decode   per layer: one call that attends and appends the new token (the
           wave that consumes the token's block patches it into its operands
           and writes it to the pool afterwards); with fuse_append=False an
           append call (ring or pages) precedes a decode call that reads the
           query's own K/V from the pool;
  prefill  per layer: attend over pool history + the chunk, then append the
           chunk (SWA chunks longer than one token would overwrite ring
           slots their first queries still need).
"""

from __future__ import annotations

import ctypes
from dataclasses import dataclass

import torch

from . import _lib
from .api import (
    FullPagePool,
    HeadShape,
    KvView,
    SwaRingPool,
    _check,
    _in_dtype,
    hybrid_attn_workspace_size,
)

SWA, FULL = "swa", "full"
GROUP_KINDS = (SWA,) * 6 + (FULL,)


@dataclass
class Layer:
    kind: str
    pool: object
    view: KvView


class HybridGroup:
    """Pools and index tables of one layer group for a fixed batch."""

    def __init__(self, shape: HeadShape, ring_id: torch.Tensor, num_rings: int, page_table: torch.Tensor,
                 num_pages: int, kinds=GROUP_KINDS, fill: float | None = None, kv_dtype: str = "bf16",
                 pools: dict | None = None):
        """pools (optional): layer index -> an existing pool of the right kind
        to use for that layer instead of a new allocation (copies of a group
        that share one layer's pool)."""
        self.shape = shape
        self.kv_dtype = kv_dtype
        self.kinds = tuple(kinds)
        self.device = ring_id.device
        self.ring_id = ring_id
        self.page_table = page_table
        self.layers = []
        pools = pools or {}
        for li, kind in enumerate(self.kinds):
            if kind == SWA:
                pool = pools[li] if li in pools else SwaRingPool(shape, num_rings, self.device, fill, kv_dtype)
                if not isinstance(pool, SwaRingPool):
                    raise ValueError(f"layer {li} needs an SWA ring pool")
                view = pool.view(ring_id)
            elif kind == FULL:
                pool = pools[li] if li in pools else FullPagePool(shape, num_pages, self.device, fill, kv_dtype)
                if not isinstance(pool, FullPagePool):
                    raise ValueError(f"layer {li} needs a Full page pool")
                view = pool.view(page_table)
            else:
                raise ValueError(f"unknown layer kind {kind!r}")
            self.layers.append(Layer(kind, pool, view))

    @property
    def batch(self) -> int:
        return int(self.ring_id.shape[0])

    def pool_bytes(self) -> dict:
        out = {SWA: 0, FULL: 0}
        for layer in self.layers:
            out[layer.kind] += layer.pool.nbytes
        return out


class _Call:
    """One library call with pre-marshalled arguments; the stream is appended at run time."""

    __slots__ = ("fn", "args", "keep")

    def __init__(self, fn, args, keep):
        self.fn = fn
        self.args = args
        self.keep = keep   # ctypes structs and every tensor whose address is in args

    def __call__(self, stream_ptr):
        st = self.fn(*self.args, stream_ptr)
        if st != _lib.HA_OK:
            _lib.check(st)


class Plan:
    """A prepared sequence of library calls (one decode step or one prefill chunk)."""

    def __init__(self, calls, labels):
        self.calls = calls
        self.labels = labels

    def run(self, stream=None):
        s = torch.cuda.current_stream() if stream is None else stream
        ptr = ctypes.c_void_p(s.cuda_stream)
        for call in self.calls:
            call(ptr)

    def run_timed(self, events, stream=None):
        """Run with a start/end event pair around each call: events[i] = (start, end)."""
        s = torch.cuda.current_stream() if stream is None else stream
        ptr = ctypes.c_void_p(s.cuda_stream)
        for call, (e0, e1) in zip(self.calls, events):
            e0.record(s)
            call(ptr)
            e1.record(s)


def _append_call(lib, shape, layer, pos0, cu_new, k_new, v_new):
    c_shape, c_view = shape.c(), layer.view.c()
    fn = lib.swa_ring_append if layer.kind == SWA else lib.full_pool_append
    dt = _in_dtype(k_new, v_new)
    args = (ctypes.byref(c_shape), ctypes.byref(c_view), pos0.data_ptr(), cu_new.data_ptr(),
            layer.view.batch, int(k_new.shape[0]), k_new.data_ptr(), v_new.data_ptr(), dt)
    return _Call(fn, args, (c_shape, c_view, layer.view, pos0, cu_new, k_new, v_new))


def plan_decode(group: HybridGroup, q, k_new, v_new, pos, kv_len, max_kv_len: int, out, lse,
                num_splits: int = 0, fuse_append: bool = True) -> Plan:
    """Decode step over every layer: q/out/lse/k_new/v_new are per-layer lists of
    [B, Hq, D] / [B, Hkv, D] tensors; pos [B] is the new token's position and
    kv_len [B] = pos + 1. With fuse_append each layer is one call that appends
    the new token and attends; otherwise an append call precedes each decode."""
    lib = _lib.load()
    shape = group.shape
    b, hq, hkv, d = group.batch, shape.num_q_heads, shape.num_kv_heads, shape.head_dim
    dev = group.device
    _check(pos, "pos", (b,), torch.int32, dev)
    _check(kv_len, "kv_len", (b,), torch.int32, dev)
    cu_one = torch.arange(b + 1, dtype=torch.int32, device=dev)
    calls, labels = [], []
    for li, layer in enumerate(group.layers):
        _check(q[li], "q", (b, hq, d), None, dev)
        _check(k_new[li], "k_new", (b, hkv, d), None, dev)
        _check(v_new[li], "v_new", (b, hkv, d), None, dev)
        _check(out[li], "out", (b, hq, d), torch.float32, dev)
        _check(lse[li], "lse", (b, hq), torch.float32, dev)
        if not fuse_append:
            calls.append(_append_call(lib, shape, layer, pos, cu_one, k_new[li], v_new[li]))
            labels.append(f"append[{li}:{layer.kind}]")
        kind = _lib.HA_SWA if layer.kind == SWA else _lib.HA_FULL
        need = hybrid_attn_workspace_size(shape, kind, True, b, max_kv_len, num_splits)
        ws = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)
        c_shape, c_view = shape.c(), layer.view.c()
        kp = k_new[li].data_ptr() if fuse_append else None
        vp = v_new[li].data_ptr() if fuse_append else None
        args = (ctypes.byref(c_shape), ctypes.byref(c_view), kv_len.data_ptr(), b, int(max_kv_len),
                q[li].data_ptr(), kp, vp, _in_dtype(q[li], k_new[li], v_new[li]), out[li].data_ptr(),
                lse[li].data_ptr(), int(num_splits), ws.data_ptr() if need else None, need)
        calls.append(_Call(lib.hybrid_attn_decode, args,
                           (c_shape, c_view, layer.view, ws, kv_len, pos, cu_one, q[li], k_new[li], v_new[li],
                            out[li], lse[li])))
        labels.append(f"decode[{li}:{layer.kind}]")
    return Plan(calls, labels)


def plan_verify(group: HybridGroup, q, k_new, v_new, kv_len, max_kv_len: int, out, lse,
                num_splits: int = 0) -> Plan:
    """Multi-token verify step over every layer: per-layer lists of
    q [B, nq, Hq, D], k_new/v_new [B, nq, Hkv, D], out [B, nq, Hq, D],
    lse [B, nq, Hq]; kv_len [B] includes the nq new tokens. Each layer is
    one call that attends and then appends the nq tokens."""
    lib = _lib.load()
    shape = group.shape
    b, hq, hkv, d = group.batch, shape.num_q_heads, shape.num_kv_heads, shape.head_dim
    dev = group.device
    _check(kv_len, "kv_len", (b,), torch.int32, dev)
    calls, labels = [], []
    for li, layer in enumerate(group.layers):
        nq = int(q[li].shape[1])
        _check(q[li], "q", (b, nq, hq, d), None, dev)
        _check(k_new[li], "k_new", (b, nq, hkv, d), None, dev)
        _check(v_new[li], "v_new", (b, nq, hkv, d), None, dev)
        _check(out[li], "out", (b, nq, hq, d), torch.float32, dev)
        _check(lse[li], "lse", (b, nq, hq), torch.float32, dev)
        kind = _lib.HA_SWA if layer.kind == SWA else _lib.HA_FULL
        c_shape, c_view = shape.c(), layer.view.c()
        need = int(lib.hybrid_attn_verify_workspace_size(ctypes.byref(c_shape), kind, b, int(max_kv_len), nq,
                                                         int(num_splits)))
        ws = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)
        args = (ctypes.byref(c_shape), ctypes.byref(c_view), kv_len.data_ptr(), b, int(max_kv_len), nq,
                q[li].data_ptr(), k_new[li].data_ptr(), v_new[li].data_ptr(),
                _in_dtype(q[li], k_new[li], v_new[li]), out[li].data_ptr(), lse[li].data_ptr(), int(num_splits),
                ws.data_ptr() if need else None, need)
        calls.append(_Call(lib.hybrid_attn_verify, args,
                           (c_shape, c_view, layer.view, ws, kv_len, q[li], k_new[li], v_new[li], out[li], lse[li])))
        labels.append(f"verify[{li}:{layer.kind}]")
    return Plan(calls, labels)


def plan_prefill(group: HybridGroup, q, k_new, v_new, hist_len, cu_new, max_new: int, out, lse) -> Plan:
    """Prefill one chunk per sequence through every layer: per-layer lists of
    q [T, Hq, D], k_new/v_new [T, Hkv, D], out [T, Hq, D], lse [T, Hq];
    hist_len [B] tokens already cached, cu_new [B+1] row offsets."""
    lib = _lib.load()
    shape = group.shape
    b, hq, hkv, d = group.batch, shape.num_q_heads, shape.num_kv_heads, shape.head_dim
    dev = group.device
    _check(hist_len, "hist_len", (b,), torch.int32, dev)
    _check(cu_new, "cu_new", (b + 1,), torch.int32, dev)
    calls, labels = [], []
    # one staging workspace serves every layer: the calls run in stream order
    t_max = max(int(x.shape[0]) for x in q)
    need = hybrid_attn_workspace_size(shape, _lib.HA_FULL, False, b, t_max)
    ws = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)
    for li, layer in enumerate(group.layers):
        t = int(q[li].shape[0])
        _check(q[li], "q", (t, hq, d), None, dev)
        _check(k_new[li], "k_new", (t, hkv, d), None, dev)
        _check(v_new[li], "v_new", (t, hkv, d), None, dev)
        _check(out[li], "out", (t, hq, d), torch.float32, dev)
        _check(lse[li], "lse", (t, hq), torch.float32, dev)
        c_shape, c_view = shape.c(), layer.view.c()
        args = (ctypes.byref(c_shape), ctypes.byref(c_view), hist_len.data_ptr(), cu_new.data_ptr(), b, t,
                int(max_new), q[li].data_ptr(), k_new[li].data_ptr(), v_new[li].data_ptr(),
                _in_dtype(q[li], k_new[li], v_new[li]), out[li].data_ptr(), lse[li].data_ptr(), ws.data_ptr(),
                ws.numel())
        calls.append(_Call(lib.hybrid_attn_prefill, args,
                           (c_shape, c_view, layer.view, ws, hist_len, cu_new, q[li], k_new[li], v_new[li],
                            out[li], lse[li])))
        labels.append(f"prefill[{li}:{layer.kind}]")
        calls.append(_append_call(lib, shape, layer, hist_len, cu_new, k_new[li], v_new[li]))
        labels.append(f"append[{li}:{layer.kind}]")
    return Plan(calls, labels)


# ---------------------------------------------------------------------------
# Layer-wise restore of cached prefix KV from pinned host memory, overlapped
# with attention (blog.hotdry.top 2026-06-09 "三层 KVCache 系统": the reused
# prefix's KV sits in a host-memory tier and is brought back layer by layer
# while earlier layers compute; youleyou.com "KVCache系统重构：让缓存真正省下来"
# for the two pools it is restored into).

class HostKv:
    """A batch's cached-prefix K/V in pinned host memory, per layer: the
    token-major rows [n, Hkv, D] (bf16) of the positions the layer restores --
    every reused position [0, L) for the full layer, the ring's window
    [max(0, L - W), L) for SWA layers -- with each sequence's first position
    and row count."""

    def __init__(self, group: HybridGroup, first, counts, k_rows, v_rows):
        self.first, self.counts, self.k, self.v = [], [], [], []
        for li in range(len(group.layers)):
            n = int(sum(int(c) for c in counts[li]))
            for name, t in (("k_rows", k_rows[li]), ("v_rows", v_rows[li])):
                if tuple(t.shape) != (n, group.shape.num_kv_heads, group.shape.head_dim) or t.dtype != torch.bfloat16:
                    raise ValueError(f"layer {li} {name}: expected bf16 [{n}, Hkv, D], got {t.dtype} {tuple(t.shape)}")
            # new pinned allocations (never registration of existing memory)
            self.k.append(k_rows[li].cpu().pin_memory())
            self.v.append(v_rows[li].cpu().pin_memory())
            self.first.append([int(x) for x in first[li]])
            self.counts.append([int(x) for x in counts[li]])

    def nbytes(self) -> int:
        return sum(t.numel() * t.element_size() for t in self.k + self.v)


class RestorePlan:
    """Per layer: a host-to-device copy of the layer's rows into a device
    staging buffer, then the library's append call scattering them into the
    layer's pool (ring slots or pages). Restores of one stack run on one copy
    stream, so groups may share staging buffers (``staging_from``): the copy
    into a buffer is queued behind the append that last read it."""

    def __init__(self, group: HybridGroup, host: HostKv, staging_from: "RestorePlan | None" = None):
        lib = _lib.load()
        dev = group.device
        self.layers = []
        for li, layer in enumerate(group.layers):
            n = host.k[li].shape[0]
            if n == 0:
                self.layers.append(None)
                continue
            shared = staging_from.layers[li] if staging_from is not None else None
            if shared is not None and tuple(shared[2].shape) == tuple(host.k[li].shape):
                k_dev, v_dev = shared[2], shared[3]
            else:
                k_dev = torch.empty_like(host.k[li], device=dev)
                v_dev = torch.empty_like(host.v[li], device=dev)
            pos0 = torch.as_tensor(host.first[li], dtype=torch.int32, device=dev)
            cu = torch.as_tensor([0] + list(_cumsum(host.counts[li])), dtype=torch.int32, device=dev)
            call = _append_call(lib, group.shape, layer, pos0, cu, k_dev, v_dev)
            self.layers.append((host.k[li], host.v[li], k_dev, v_dev, call))

    def run_layer(self, li: int, stream) -> None:
        item = self.layers[li]
        if item is None:
            return
        k_host, v_host, k_dev, v_dev, call = item
        with torch.cuda.stream(stream):
            k_dev.copy_(k_host, non_blocking=True)
            v_dev.copy_(v_host, non_blocking=True)
        call(ctypes.c_void_p(stream.cuda_stream))

    def run(self, stream) -> None:
        for li in range(len(self.layers)):
            self.run_layer(li, stream)


def _cumsum(xs):
    s = 0
    for x in xs:
        s += x
        yield s


def layer_calls(plan: Plan, num_layers: int):
    """A group's prefill plan split by layer (labels carry the layer index)."""
    by_layer = [[] for _ in range(num_layers)]
    for call, label in zip(plan.calls, plan.labels):
        by_layer[int(label.split("[", 1)[1].split(":", 1)[0])].append(call)
    return by_layer


def run_restore_overlapped(restores, prefills, compute_stream, copy_stream) -> None:
    """A stack of groups (layers in forward order, group by group): every
    layer's restore is queued on the copy stream up front, and each layer's
    prefill (with its chunk append) waits only for its own restore, so layer
    l+1's copy runs while layer l computes. The restores start after
    everything already queued on the compute stream, so a repeated run cannot
    overwrite a pool an earlier run still reads."""
    if isinstance(restores, RestorePlan):
        restores, prefills = [restores], [prefills]
    if len(restores) != len(prefills):
        raise ValueError("one restore plan per prefill plan")
    copy_stream.wait_stream(compute_stream)
    steps = []
    for restore, plan in zip(restores, prefills):
        nl = len(restore.layers)
        for li, calls in enumerate(layer_calls(plan, nl)):
            restore.run_layer(li, copy_stream)
            ev = torch.cuda.Event()
            ev.record(copy_stream)
            steps.append((ev, calls))
    ptr = ctypes.c_void_p(compute_stream.cuda_stream)
    for ev, calls in steps:
        compute_stream.wait_event(ev)
        for call in calls:
            call(ptr)
    # the staging buffers and pools are reused by the next run: make later
    # work on the copy stream wait for this run's compute
    copy_stream.wait_stream(compute_stream)
