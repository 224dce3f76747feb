"""Seeded synthetic inputs shared by the tests, the smoke run and the bench.

This module holds no attention or indexing arithmetic: it only draws the
workloads' structure (lengths, evictions, physical page order, ring ids,
token ids) with NumPy and the value tensors (Q/K/V ~ N(0,1), drawn in
float32 and rounded to bfloat16) with a seeded torch generator. Both the
oracle side and the HIP side consume exactly these arrays.

Workloads (all W = 128, 16-token pages, 6:1 SWA:full layer groups as the
pages describe them -- htx.com news section 工程一; blog.hotdry.top
2026-06-09 sections "Hybrid SWA：用 1/7 计算量捕获长程依赖" and "生产级调参清单"):

  small    1 sequence of 512 tokens, one SWA + one full layer, Hq/Hkv/D = 4/1/64,
           float32 inputs, scale 1/8; prefill then 16 decode steps.
  decode   64 sequences x 8192 cached tokens, one 7-layer group, Hq/Hkv/D = 64/8/128.
  chunked  4 sequences x 32768 tokens prefilled in 8192-token chunks.
  reuse    32 sequences: cached prefix P ~ U{4096..65536}, a fraction f ~ U[0, 0.30)
           of the last 128 SWA slots evicted, suffix S ~ U{512..2048}.
  ragged   24 sequences of cached lengths from three buckets
           (12 x U{1K..64K}, 8 x U{64K..256K}, 4 x U{256K..1M}), the length
           buckets named in blog.hotdry.top 2026-06-09 "PD 分离与长度分桶".
"""

from .workloads import (  # noqa: F401
    BIG_SHAPE,
    GROUP_KINDS,
    K_VALUES,
    PAGE,
    Q_VALUES,
    SMALL_SHAPE,
    V_VALUES,
    WINDOW,
    HeadShape,
    Structure,
    allocate_pages,
    allocate_rings,
    chunked_structure,
    decode_structure,
    normal_bf16,
    normal_f32,
    ragged_structure,
    reuse_structure,
    reuse_tokens,
    small_structure,
)
