"""ctypes declarations of the C ABI in include/hybrid_attn.h, include/prefix_tree.h and include/ha_probe.h.

Loading fails loudly when libhybridattn.so has not been built: there is no
fallback implementation.
"""

from __future__ import annotations

import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libhybridattn.so")

HA_OK = 0
HA_ERR_NULL = 1
HA_ERR_SHAPE = 2
HA_ERR_RANGE = 3
HA_ERR_WORKSPACE = 4
HA_ERR_UNSUPPORTED = 5
HA_ERR_HIP = 6

HA_BF16 = 0
HA_F32 = 1
HA_SWA = 0
HA_FULL = 1
HA_KV_BF16 = 0
HA_KV_INT8 = 1

ABI_VERSION = 8

# Bytes of the library-owned scratch array of hybrid_attn_decode_noalloc.
HA_DECODE_SCRATCH_BYTES = 64 << 20

# Every symbol include/*.h declares.
EXPORTS = (
    "swa_ring_append",
    "full_pool_append",
    "swa_ring_read",
    "full_pool_read",
    "window_safe_match",
    "hybrid_attn_prefill",
    "hybrid_attn_decode",
    "hybrid_attn_decode_noalloc",
    "hybrid_attn_workspace_size",
    "hybrid_attn_decode_splits",
    "hybrid_attn_verify",
    "hybrid_attn_verify_workspace_size",
    "ha_status_str",
    "ha_last_error",
    "ha_abi_version",
    "ha_tree_create",
    "ha_tree_destroy",
    "ha_tree_insert",
    "ha_tree_match",
    "ha_tree_lock",
    "ha_tree_ring_advance",
    "ha_tree_ring_release",
    "ha_tree_evict_full",
    "ha_tree_evict_swa",
    "ha_tree_stats",
    "ha_probe_paged_read",
    "ha_probe_mfma_bf16",
    "ha_probe_coissue",
)


class HaShape(ctypes.Structure):
    _fields_ = [
        ("num_q_heads", ctypes.c_int32),
        ("num_kv_heads", ctypes.c_int32),
        ("head_dim", ctypes.c_int32),
        ("window", ctypes.c_int32),
        ("page_size", ctypes.c_int32),
        ("softmax_scale", ctypes.c_float),
    ]


class HaKvView(ctypes.Structure):
    _fields_ = [
        ("kind", ctypes.c_int32),
        ("k", ctypes.c_void_p),
        ("v", ctypes.c_void_p),
        ("num_blocks", ctypes.c_int32),
        ("table", ctypes.c_void_p),
        ("table_stride", ctypes.c_int32),
        ("kv_dtype", ctypes.c_int32),
        ("k_scale", ctypes.c_void_p),
        ("v_scale", ctypes.c_void_p),
    ]


class HybridAttnError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"{status_str(status)}: {message}")
        self.status = status


_lib = None


def load() -> ctypes.CDLL:
    """Load libhybridattn.so (once) and declare the ABI."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise ImportError(
            f"{LIB_PATH} is missing: build the HIP library first "
            "(python -m hybrid_sliding_window_gqa_amd.build)"
        )
    lib = ctypes.CDLL(LIB_PATH)
    p, i32, i64, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t
    shp, view = ctypes.POINTER(HaShape), ctypes.POINTER(HaKvView)
    append_args = [shp, view, p, p, i32, i32, p, p, i32, p]
    lib.swa_ring_append.argtypes = append_args
    lib.full_pool_append.argtypes = append_args
    lib.swa_ring_read.argtypes = [shp, view, p, p, i32, i32, p, p, p]
    lib.full_pool_read.argtypes = [shp, view, p, p, i32, i32, p, p, p]
    lib.window_safe_match.argtypes = [p, i64, p, i64, p, i32, ctypes.POINTER(i64)]
    lib.hybrid_attn_prefill.argtypes = [shp, view, p, p, i32, i32, i32, p, p, p, i32, p, p, p, sz, p]
    lib.hybrid_attn_decode.argtypes = [shp, view, p, i32, i32, p, p, p, i32, p, p, i32, p, sz, p]
    lib.hybrid_attn_decode_noalloc.argtypes = [shp, view, p, i32, i32, p, p, p, i32, p, p, i32, p]
    lib.hybrid_attn_workspace_size.argtypes = [shp, i32, i32, i32, i32, i32]
    lib.hybrid_attn_workspace_size.restype = sz
    lib.hybrid_attn_decode_splits.argtypes = [shp, i32, i32, i32, i32]
    lib.hybrid_attn_decode_splits.restype = i32
    lib.hybrid_attn_verify.argtypes = [shp, view, p, i32, i32, i32, p, p, p, i32, p, p, i32, p, sz, p]
    lib.hybrid_attn_verify_workspace_size.argtypes = [shp, i32, i32, i32, i32, i32]
    lib.hybrid_attn_verify_workspace_size.restype = sz
    for fn in ("swa_ring_append", "full_pool_append", "swa_ring_read", "full_pool_read", "window_safe_match",
               "hybrid_attn_prefill",
               "hybrid_attn_decode", "hybrid_attn_decode_noalloc", "hybrid_attn_verify"):
        getattr(lib, fn).restype = i32
    lib.ha_status_str.argtypes = [i32]
    lib.ha_status_str.restype = ctypes.c_char_p
    lib.ha_last_error.argtypes = []
    lib.ha_last_error.restype = ctypes.c_char_p
    lib.ha_abi_version.argtypes = []
    lib.ha_abi_version.restype = i32
    pi64 = ctypes.POINTER(i64)
    tree_fns = {
        "ha_tree_create": [i32, i32, ctypes.POINTER(p)],
        "ha_tree_insert": [p, p, i64, p, i32, i64, i32, p, p],
        "ha_tree_match": [p, p, i64, pi64, p, p, p],
        "ha_tree_lock": [p, p, i64, i32],
        "ha_tree_ring_advance": [p, i32, i64],
        "ha_tree_ring_release": [p, i32],
        "ha_tree_evict_full": [p, i64, p, i64, pi64, p, i64, pi64],
        "ha_tree_evict_swa": [p, i64, p, i64, pi64],
        "ha_tree_stats": [p, p],
    }
    for fn, args in tree_fns.items():
        getattr(lib, fn).argtypes = args
        getattr(lib, fn).restype = i32
    lib.ha_probe_paged_read.argtypes = [shp, view, p, i32, p, i32, p]
    lib.ha_probe_paged_read.restype = i32
    lib.ha_probe_mfma_bf16.argtypes = [i32, i32, p, p]
    lib.ha_probe_mfma_bf16.restype = i32
    lib.ha_probe_coissue.argtypes = [i32, i32, i32, p, p]
    lib.ha_probe_coissue.restype = i32
    lib.ha_tree_destroy.argtypes = [p]
    lib.ha_tree_destroy.restype = None
    if lib.ha_abi_version() != ABI_VERSION:
        raise ImportError(f"libhybridattn.so ABI {lib.ha_abi_version()} != binding ABI {ABI_VERSION}")
    _lib = lib
    return lib


def status_str(status: int) -> str:
    return load().ha_status_str(int(status)).decode()


def check(status: int) -> None:
    if status != HA_OK:
        raise HybridAttnError(status, load().ha_last_error().decode())
