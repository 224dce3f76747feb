"""Oracle: 8-bit KV quantization, by its definition (test infrastructure only).

The pages list low-bit KV storage among the ways to cut the bytes decode reads
(blog.hotdry.top 2026-06-12, section "KV Cache 量化策略的技术选型") without
fixing a format. The reading used here (the plainest one that needs no codec):
symmetric INT8 with one scale per (token, kv head) row of D channels,

    amax  = max_d |x_d|                      (x: the row as bf16 values)
    scale = amax / 127                       (IEEE float32 division)
    q_d   = clamp(rint(x_d / scale), -127, 127)   (float32 division, ties to even)
    scale = 0 and q = 0 for an all-zero row,

and the dequantized value is q_d * scale. Every quantised code is decided in
float32, the precision the kernels use, so codes and scales are reproduced
bit for bit. float32 inputs are first rounded to bf16 (the pools' input
rounding).
"""

from __future__ import annotations

import numpy as np


def bf16_round(x) -> np.ndarray:
    """Round float32 values to bfloat16 (nearest, ties to even), returned as float32."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    r = (u + 0x7FFF + ((u >> 16) & 1)) & 0xFFFF0000
    return r.astype(np.uint32).view(np.float32)


def quantize_rows(x):
    """x [..., D] float32 (already bf16 values) -> (codes int8 [..., D], scale float32 [...])."""
    x = np.asarray(x, dtype=np.float32)
    amax = np.max(np.abs(x), axis=-1)
    scale = (amax / np.float32(127.0)).astype(np.float32)
    safe = np.where(scale > 0, scale, np.float32(1.0)).astype(np.float32)
    ratio = (x / safe[..., None]).astype(np.float32)
    codes = np.clip(np.rint(ratio), -127, 127)
    codes = np.where(scale[..., None] > 0, codes, 0).astype(np.int8)
    return codes, scale


def dequantize_rows(codes, scale) -> np.ndarray:
    """Exact dequantized values (float64)."""
    return np.asarray(codes, dtype=np.float64) * np.asarray(scale, dtype=np.float64)[..., None]
