"""Python binding of the C ABI: same names, argument marshalling only.

Each function checks that the tensors it is handed have the shapes, dtypes,
devices and contiguity the C ABI documents (the C side cannot see buffer
sizes), converts them to raw pointers and calls libhybridattn.so on the
current HIP stream. Every step of the computation runs in the library's
kernels; nothing here computes attention.
"""

from __future__ import annotations

import ctypes
from dataclasses import dataclass

import numpy as np
import torch

from . import _lib
from ._lib import HA_BF16, HA_F32, HA_FULL, HA_KV_BF16, HA_KV_INT8, HA_SWA, HaKvView, HaShape, check, load

BLOCK = 16


@dataclass(frozen=True)
class HeadShape:
    """Head geometry of a layer stack (ha_shape)."""

    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    window: int = 128
    page_size: int = 16
    softmax_scale: float = 0.0  # <= 0: 1/sqrt(head_dim)

    def c(self) -> HaShape:
        return HaShape(self.num_q_heads, self.num_kv_heads, self.head_dim, self.window,
                       self.page_size, float(self.softmax_scale))

    @property
    def group(self) -> int:
        return self.num_q_heads // self.num_kv_heads


@dataclass
class KvView:
    """One layer's pool plus the per-sequence index that addresses it (ha_kv_view)."""

    kind: int
    k: torch.Tensor
    v: torch.Tensor
    num_blocks: int
    table: torch.Tensor          # ring ids [B] or page table [B, stride], int32
    table_stride: int = 0
    kv_dtype: int = HA_KV_BF16   # HA_KV_INT8: k/v hold int8 codes, scales below
    k_scale: torch.Tensor | None = None
    v_scale: torch.Tensor | None = None

    def c(self) -> HaKvView:
        ks = self.k_scale.data_ptr() if self.k_scale is not None else None
        vs = self.v_scale.data_ptr() if self.v_scale is not None else None
        return HaKvView(self.kind, self.k.data_ptr(), self.v.data_ptr(), self.num_blocks,
                        self.table.data_ptr(), self.table_stride, self.kv_dtype, ks, vs)

    @property
    def batch(self) -> int:
        return int(self.table.shape[0])


class _PoolStorage:
    """K/V blocks of one layer in the pool format: bfloat16, or int8 codes
    with one float32 scale per (block, kv head, token) for K and for V
    (include/hybrid_attn.h). fill (tests): bf16 values, or int8 scales (the
    codes then hold 127), so an unwritten slot shows up if it is ever used."""

    def _alloc(self, lead, d, device, kv_dtype: str, fill):
        if kv_dtype not in ("bf16", "int8"):
            raise ValueError(f"kv_dtype must be 'bf16' or 'int8', got {kv_dtype!r}")
        self.kv_dtype = HA_KV_INT8 if kv_dtype == "int8" else HA_KV_BF16
        dt = torch.int8 if kv_dtype == "int8" else torch.bfloat16
        self.k = torch.empty(*lead, BLOCK * d, dtype=dt, device=device)
        self.v = torch.empty(*lead, BLOCK * d, dtype=dt, device=device)
        self.k_scale = self.v_scale = None
        if kv_dtype == "int8":
            self.k_scale = torch.empty(*lead, BLOCK, dtype=torch.float32, device=device)
            self.v_scale = torch.empty(*lead, BLOCK, dtype=torch.float32, device=device)
        if fill is not None:
            if kv_dtype == "int8":
                self.k.fill_(127)
                self.v.fill_(127)
                self.k_scale.fill_(fill)
                self.v_scale.fill_(fill)
            else:
                self.k.fill_(fill)
                self.v.fill_(fill)

    def _view(self, kind, num_blocks, table, stride) -> KvView:
        return KvView(kind, self.k, self.v, num_blocks, table, stride, self.kv_dtype, self.k_scale, self.v_scale)

    @property
    def nbytes(self) -> int:
        n = self.k.numel() * self.k.element_size() + self.v.numel() * self.v.element_size()
        if self.k_scale is not None:
            n += (self.k_scale.numel() + self.v_scale.numel()) * 4
        return n


class SwaRingPool(_PoolStorage):
    """SWA pool of one layer: W slots per (ring, kv head).

    K and V are [rings, Hkv, ceil(W/16), 16*D]: 16-slot blocks stored in the
    library's matrix-core operand order (include/hybrid_attn.h), the last
    block's slots past W unused; int8 pools add k_scale / v_scale
    [rings, Hkv, ceil(W/16), 16]."""

    def __init__(self, shape: HeadShape, num_rings: int, device, fill: float | None = None,
                 kv_dtype: str = "bf16"):
        w, d, h = shape.window, shape.head_dim, shape.num_kv_heads
        self.shape = shape
        self.num_rings = num_rings
        self._alloc((num_rings, h, -(-w // BLOCK)), d, device, kv_dtype, fill)

    def view(self, ring_id: torch.Tensor) -> KvView:
        _check_table(ring_id, 1, self.k.device)
        return self._view(HA_SWA, self.num_rings, ring_id, 0)


class FullPagePool(_PoolStorage):
    """Full pool of one layer: pages of shape.page_size tokens (16, 32, ...).

    K and V are [pages, Hkv, page_size/16, 16*D]: each page holds
    page_size/16 16-token blocks per kv head in the library's matrix-core
    operand order (include/hybrid_attn.h); int8 pools add k_scale / v_scale
    [pages, Hkv, page_size/16, 16]."""

    def __init__(self, shape: HeadShape, num_pages: int, device, fill: float | None = None,
                 kv_dtype: str = "bf16"):
        d, h = shape.head_dim, shape.num_kv_heads
        ps = shape.page_size
        if ps < BLOCK or ps & (ps - 1):
            raise ValueError(f"page_size must be a power of two >= {BLOCK}, got {shape.page_size}")
        self.shape = shape
        self.num_pages = num_pages
        self._alloc((num_pages, h, shape.page_size // BLOCK), d, device, kv_dtype, fill)

    def view(self, page_table: torch.Tensor) -> KvView:
        _check_table(page_table, 2, self.k.device)
        return self._view(HA_FULL, self.num_pages, page_table, int(page_table.shape[1]))


class PageAllocator:
    """Host-side free list of physical page ids: the Full pool grows on demand
    by handing out more pages as sequences get longer."""

    def __init__(self, num_pages: int, order=None):
        ids = list(range(num_pages)) if order is None else [int(x) for x in order]
        if sorted(ids) != list(range(num_pages)):
            raise ValueError("order must be a permutation of range(num_pages)")
        self._free = ids[::-1]

    @property
    def free(self) -> int:
        return len(self._free)

    def alloc(self, count: int) -> list:
        if count > len(self._free):
            raise MemoryError(f"Full pool exhausted: need {count} pages, {len(self._free)} free")
        return [self._free.pop() for _ in range(count)]

    def release(self, pages) -> None:
        self._free.extend(int(p) for p in reversed(list(pages)))


def _stream_ptr(stream) -> ctypes.c_void_p:
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def _check_table(t: torch.Tensor, ndim: int, device) -> None:
    if t.dtype != torch.int32 or t.dim() != ndim or not t.is_contiguous():
        raise ValueError(f"index table must be a contiguous int32 tensor with {ndim} dims")
    if t.device != device:
        raise ValueError("index table and pool are on different devices")


def _in_dtype(*ts: torch.Tensor) -> int:
    dt = ts[0].dtype
    if any(t.dtype != dt for t in ts):
        raise ValueError("inputs must share one dtype")
    if dt == torch.bfloat16:
        return HA_BF16
    if dt == torch.float32:
        return HA_F32
    raise ValueError(f"unsupported input dtype {dt}")


def _check(t: torch.Tensor, name: str, shape, dtype=None, device=None) -> None:
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    if device is not None and t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")


def _append(fn, shape: HeadShape, view: KvView, pos0, cu_new, k_new, v_new, stream):
    dev = view.k.device
    b = view.batch
    _check(pos0, "pos0", (b,), torch.int32, dev)
    _check(cu_new, "cu_new", (b + 1,), torch.int32, dev)
    t = int(k_new.shape[0])
    _check(k_new, "k_new", (t, shape.num_kv_heads, shape.head_dim), None, dev)
    _check(v_new, "v_new", (t, shape.num_kv_heads, shape.head_dim), None, dev)
    dt = _in_dtype(k_new, v_new)
    c_shape, c_view = shape.c(), view.c()
    check(fn(ctypes.byref(c_shape), ctypes.byref(c_view), pos0.data_ptr(), cu_new.data_ptr(), b, t,
             k_new.data_ptr(), v_new.data_ptr(), dt, _stream_ptr(stream)))


def swa_ring_append(shape: HeadShape, ring: KvView, pos0: torch.Tensor, cu_new: torch.Tensor,
                    k_new: torch.Tensor, v_new: torch.Tensor, stream=None) -> None:
    """Write new K/V rows into the SWA ring pool (slot = position mod W)."""
    if ring.kind != HA_SWA:
        raise ValueError("swa_ring_append needs an SWA ring view")
    _append(load().swa_ring_append, shape, ring, pos0, cu_new, k_new, v_new, stream)


def full_pool_append(shape: HeadShape, pages: KvView, pos0: torch.Tensor, cu_new: torch.Tensor,
                     k_new: torch.Tensor, v_new: torch.Tensor, stream=None) -> None:
    """Write new K/V rows into the Full page pool through the page table."""
    if pages.kind != HA_FULL:
        raise ValueError("full_pool_append needs a Full page view")
    _append(load().full_pool_append, shape, pages, pos0, cu_new, k_new, v_new, stream)


def _read(fn, shape: HeadShape, view: KvView, pos0, cu, k_out, v_out, stream):
    dev = view.k.device
    b = view.batch
    _check(pos0, "pos0", (b,), torch.int32, dev)
    _check(cu, "cu", (b + 1,), torch.int32, dev)
    if k_out is None or v_out is None:
        raise ValueError("k_out and v_out are required (their first dim is the row count)")
    t = int(k_out.shape[0])
    _check(k_out, "k_out", (t, shape.num_kv_heads, shape.head_dim), torch.bfloat16, dev)
    _check(v_out, "v_out", (t, shape.num_kv_heads, shape.head_dim), torch.bfloat16, dev)
    c_shape, c_view = shape.c(), view.c()
    check(fn(ctypes.byref(c_shape), ctypes.byref(c_view), pos0.data_ptr(), cu.data_ptr(), b, t, k_out.data_ptr(),
             v_out.data_ptr(), _stream_ptr(stream)))
    return k_out, v_out


def swa_ring_read(shape: HeadShape, ring: KvView, pos0: torch.Tensor, cu: torch.Tensor, k_out: torch.Tensor,
                  v_out: torch.Tensor, stream=None):
    """Copy positions pos0[b] + i out of each sequence's ring (slot = position mod W) into token-major rows."""
    if ring.kind != HA_SWA:
        raise ValueError("swa_ring_read needs an SWA ring view")
    return _read(load().swa_ring_read, shape, ring, pos0, cu, k_out, v_out, stream)


def full_pool_read(shape: HeadShape, pages: KvView, pos0: torch.Tensor, cu: torch.Tensor, k_out: torch.Tensor,
                   v_out: torch.Tensor, stream=None):
    """Copy positions pos0[b] + i out of each sequence's pages into token-major rows."""
    if pages.kind != HA_FULL:
        raise ValueError("full_pool_read needs a Full page view")
    return _read(load().full_pool_read, shape, pages, pos0, cu, k_out, v_out, stream)


def window_safe_match(req_tokens, cached_tokens, swa_valid, window: int) -> int:
    """Reusable prefix length under the window-safe rule (host call)."""
    req = np.ascontiguousarray(req_tokens, dtype=np.int32)
    cached = np.ascontiguousarray(cached_tokens, dtype=np.int32)
    valid = np.ascontiguousarray(swa_valid, dtype=np.uint8)
    if valid.shape != cached.shape:
        raise ValueError("one validity flag per cached token is required")
    out = ctypes.c_int64(-1)
    check(load().window_safe_match(req.ctypes.data, req.size, cached.ctypes.data, cached.size,
                                   valid.ctypes.data, int(window), ctypes.byref(out)))
    return int(out.value)


def hybrid_attn_workspace_size(shape: HeadShape, kind: int, decode: bool, batch: int, max_kv_len: int,
                               num_splits: int = 0) -> int:
    c_shape = shape.c()
    return int(load().hybrid_attn_workspace_size(ctypes.byref(c_shape), kind, int(bool(decode)), batch,
                                                 max_kv_len, num_splits))


def hybrid_attn_decode_splits(shape: HeadShape, kind: int, batch: int, max_kv_len: int, num_splits: int = 0) -> int:
    c_shape = shape.c()
    return int(load().hybrid_attn_decode_splits(ctypes.byref(c_shape), kind, batch, max_kv_len, num_splits))


def hybrid_attn_prefill(shape: HeadShape, kv: KvView, hist_len: torch.Tensor, cu_new: torch.Tensor,
                        q: torch.Tensor, k_new: torch.Tensor, v_new: torch.Tensor, max_new: int,
                        out: torch.Tensor | None = None, lse: torch.Tensor | None = None,
                        workspace: torch.Tensor | None = None, stream=None):
    """Causal prefill of a chunk per sequence over pool history + the chunk itself.

    Returns (out float32 [T, Hq, D], lse float32 [T, Hq])."""
    dev = kv.k.device
    b = kv.batch
    t = int(q.shape[0])
    hq, hkv, d = shape.num_q_heads, shape.num_kv_heads, shape.head_dim
    _check(hist_len, "hist_len", (b,), torch.int32, dev)
    _check(cu_new, "cu_new", (b + 1,), torch.int32, dev)
    _check(q, "q", (t, hq, d), None, dev)
    _check(k_new, "k_new", (t, hkv, d), None, dev)
    _check(v_new, "v_new", (t, hkv, d), None, dev)
    dt = _in_dtype(q, k_new, v_new)
    if out is None:
        out = torch.empty(t, hq, d, dtype=torch.float32, device=dev)
    if lse is None:
        lse = torch.empty(t, hq, dtype=torch.float32, device=dev)
    _check(out, "out", (t, hq, d), torch.float32, dev)
    _check(lse, "lse", (t, hq), torch.float32, dev)
    need = hybrid_attn_workspace_size(shape, kv.kind, False, b, t)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)
    ws_bytes = workspace.numel() * workspace.element_size()
    c_shape, c_view = shape.c(), kv.c()
    check(load().hybrid_attn_prefill(ctypes.byref(c_shape), ctypes.byref(c_view), hist_len.data_ptr(),
                                     cu_new.data_ptr(), b, t, int(max_new), q.data_ptr(), k_new.data_ptr(),
                                     v_new.data_ptr(), dt, out.data_ptr(), lse.data_ptr(), workspace.data_ptr(),
                                     ws_bytes, _stream_ptr(stream)))
    return out, lse


def hybrid_attn_decode(shape: HeadShape, kv: KvView, kv_len: torch.Tensor, q: torch.Tensor, max_kv_len: int,
                       out: torch.Tensor | None = None, lse: torch.Tensor | None = None, num_splits: int = 0,
                       workspace: torch.Tensor | None = None, stream=None, k_new: torch.Tensor | None = None,
                       v_new: torch.Tensor | None = None):
    """Decode one query per sequence at position kv_len - 1 over the pool.

    Without k_new/v_new the query's own K/V must already be in the pool. With
    them ([B, Hkv, D], same dtype as q) the call also appends that token, in
    the same launch.

    Returns (out float32 [B, Hq, D], lse float32 [B, Hq])."""
    dev = kv.k.device
    b = kv.batch
    hq, d = shape.num_q_heads, shape.head_dim
    _check(kv_len, "kv_len", (b,), torch.int32, dev)
    _check(q, "q", (b, hq, d), None, dev)
    if (k_new is None) != (v_new is None):
        raise ValueError("pass both k_new and v_new (fused append) or neither")
    if k_new is not None:
        _check(k_new, "k_new", (b, shape.num_kv_heads, d), None, dev)
        _check(v_new, "v_new", (b, shape.num_kv_heads, d), None, dev)
        dt = _in_dtype(q, k_new, v_new)
    else:
        dt = _in_dtype(q)
    if out is None:
        out = torch.empty(b, hq, d, dtype=torch.float32, device=dev)
    if lse is None:
        lse = torch.empty(b, hq, dtype=torch.float32, device=dev)
    _check(out, "out", (b, hq, d), torch.float32, dev)
    _check(lse, "lse", (b, hq), torch.float32, dev)
    need = hybrid_attn_workspace_size(shape, kv.kind, True, b, max_kv_len, num_splits)
    if need and workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=dev)
    ws_ptr = workspace.data_ptr() if workspace is not None else None
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    c_shape, c_view = shape.c(), kv.c()
    kp = k_new.data_ptr() if k_new is not None else None
    vp = v_new.data_ptr() if v_new is not None else None
    check(load().hybrid_attn_decode(ctypes.byref(c_shape), ctypes.byref(c_view), kv_len.data_ptr(), b,
                                    int(max_kv_len), q.data_ptr(), kp, vp, dt, out.data_ptr(), lse.data_ptr(),
                                    int(num_splits), ws_ptr, ws_bytes, _stream_ptr(stream)))
    return out, lse


def hybrid_attn_decode_noalloc(shape: HeadShape, kv: KvView, kv_len: torch.Tensor, q: torch.Tensor,
                               max_kv_len: int, out: torch.Tensor, lse: torch.Tensor, num_splits: int = 0,
                               stream=None, k_new: torch.Tensor | None = None, v_new: torch.Tensor | None = None):
    """hybrid_attn_decode for callers that cannot allocate: the caller passes
    the outputs, and the split-K partials live in the library's static scratch
    array (HA_DECODE_SCRATCH_BYTES per device). Nothing is allocated here or
    in the library. Returns (out, lse)."""
    dev = kv.k.device
    b = kv.batch
    hq, d = shape.num_q_heads, shape.head_dim
    _check(kv_len, "kv_len", (b,), torch.int32, dev)
    _check(q, "q", (b, hq, d), None, dev)
    if (k_new is None) != (v_new is None):
        raise ValueError("pass both k_new and v_new (fused append) or neither")
    if k_new is not None:
        _check(k_new, "k_new", (b, shape.num_kv_heads, d), None, dev)
        _check(v_new, "v_new", (b, shape.num_kv_heads, d), None, dev)
        dt = _in_dtype(q, k_new, v_new)
    else:
        dt = _in_dtype(q)
    _check(out, "out", (b, hq, d), torch.float32, dev)
    _check(lse, "lse", (b, hq), torch.float32, dev)
    c_shape, c_view = shape.c(), kv.c()
    kp = k_new.data_ptr() if k_new is not None else None
    vp = v_new.data_ptr() if v_new is not None else None
    check(load().hybrid_attn_decode_noalloc(ctypes.byref(c_shape), ctypes.byref(c_view), kv_len.data_ptr(), b,
                                            int(max_kv_len), q.data_ptr(), kp, vp, dt, out.data_ptr(),
                                            lse.data_ptr(), int(num_splits), _stream_ptr(stream)))
    return out, lse


def hybrid_attn_verify_workspace_size(shape: HeadShape, kind: int, batch: int, max_kv_len: int, nq: int,
                                      num_splits: int = 0) -> int:
    c_shape = shape.c()
    return int(load().hybrid_attn_verify_workspace_size(ctypes.byref(c_shape), kind, batch, max_kv_len, nq,
                                                        num_splits))


def hybrid_attn_verify(shape: HeadShape, kv: KvView, kv_len: torch.Tensor, q: torch.Tensor, k_new: torch.Tensor,
                       v_new: torch.Tensor, max_kv_len: int, out: torch.Tensor | None = None,
                       lse: torch.Tensor | None = None, num_splits: int = 0, workspace: torch.Tensor | None = None,
                       stream=None):
    """Verify nq new tokens per sequence (positions kv_len - nq .. kv_len - 1),
    causal among themselves, over the pool history; then append them.

    q [B, nq, Hq, D]; k_new/v_new [B, nq, Hkv, D] (same dtype as q).
    Returns (out float32 [B, nq, Hq, D], lse float32 [B, nq, Hq])."""
    dev = kv.k.device
    b = kv.batch
    hq, hkv, d = shape.num_q_heads, shape.num_kv_heads, shape.head_dim
    if q.dim() != 4:
        raise ValueError(f"q must be [B, nq, Hq, D], got shape {tuple(q.shape)}")
    nq = int(q.shape[1])
    _check(kv_len, "kv_len", (b,), torch.int32, dev)
    _check(q, "q", (b, nq, hq, d), None, dev)
    _check(k_new, "k_new", (b, nq, hkv, d), None, dev)
    _check(v_new, "v_new", (b, nq, hkv, d), None, dev)
    dt = _in_dtype(q, k_new, v_new)
    if out is None:
        out = torch.empty(b, nq, hq, d, dtype=torch.float32, device=dev)
    if lse is None:
        lse = torch.empty(b, nq, hq, dtype=torch.float32, device=dev)
    _check(out, "out", (b, nq, hq, d), torch.float32, dev)
    _check(lse, "lse", (b, nq, hq), torch.float32, dev)
    need = hybrid_attn_verify_workspace_size(shape, kv.kind, b, max_kv_len, nq, num_splits)
    if need and workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=dev)
    ws_ptr = workspace.data_ptr() if workspace is not None else None
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    c_shape, c_view = shape.c(), kv.c()
    check(load().hybrid_attn_verify(ctypes.byref(c_shape), ctypes.byref(c_view), kv_len.data_ptr(), b,
                                    int(max_kv_len), nq, q.data_ptr(), k_new.data_ptr(), v_new.data_ptr(), dt,
                                    out.data_ptr(), lse.data_ptr(), int(num_splits), ws_ptr, ws_bytes,
                                    _stream_ptr(stream)))
    return out, lse
