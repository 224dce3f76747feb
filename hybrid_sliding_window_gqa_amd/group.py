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
  decode   per layer: append the new token (ring or pages), then attend
           (decode reads the query's own K/V from the pool);
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
                 num_pages: int, kinds=GROUP_KINDS, fill: float | None = None):
        self.shape = shape
        self.kinds = tuple(kinds)
        self.device = ring_id.device
        self.ring_id = ring_id
        self.page_table = page_table
        self.layers = []
        for kind in self.kinds:
            if kind == SWA:
                pool = SwaRingPool(shape, num_rings, self.device, fill)
                view = pool.view(ring_id)
            elif kind == FULL:
                pool = FullPagePool(shape, num_pages, self.device, fill)
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
            out[layer.kind] += layer.pool.k.numel() * 2 + layer.pool.v.numel() * 2
        return out


class _Call:
    """One library call with pre-marshalled arguments; the stream is appended at run time."""

    __slots__ = ("fn", "args", "keep")

    def __init__(self, fn, args, keep):
        self.fn = fn
        self.args = args
        self.keep = keep   # ctypes structs / tensors that must outlive the call

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
    return _Call(fn, args, (c_shape, c_view, pos0, cu_new, k_new, v_new))


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
                           (c_shape, c_view, ws, kv_len, cu_one, k_new[li], v_new[li])))
        labels.append(f"decode[{li}:{layer.kind}]")
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
        calls.append(_Call(lib.hybrid_attn_prefill, args, (c_shape, c_view, ws)))
        labels.append(f"prefill[{li}:{layer.kind}]")
        calls.append(_append_call(lib, shape, layer, hist_len, cu_new, k_new[li], v_new[li]))
        labels.append(f"append[{li}:{layer.kind}]")
    return Plan(calls, labels)
