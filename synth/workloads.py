"""Seeded structure and value generators for the five synthetic workloads.

Structure uses numpy.random.default_rng([workload_id, 0]); values use a torch
generator seeded with 1000 * workload_id + layer (+ a per-purpose offset), so
every layer's tensors are independent and reproducible on one device.
"""

from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np

WINDOW = 128
PAGE = 16

WORKLOAD_IDS = {"small": 1, "decode": 2, "chunked": 3, "reuse": 4, "ragged": 5}


@dataclass(frozen=True)
class HeadShape:
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    window: int = WINDOW
    page_size: int = PAGE
    scale: float = 0.0          # 0 selects 1/sqrt(head_dim)


SMALL_SHAPE = HeadShape(4, 1, 64)
BIG_SHAPE = HeadShape(64, 8, 128)

# Layer kinds of one 6:1 group; the full layer is the last of the seven.
GROUP_KINDS = ["swa"] * 6 + ["full"]


def structure_rng(workload: str) -> np.random.Generator:
    return np.random.default_rng([WORKLOAD_IDS[workload], 0])


def allocate_pages(rng: np.random.Generator, tokens_per_seq, page_size: int = PAGE, spare: int = 8):
    """Give each sequence enough physical pages for `tokens_per_seq` tokens.

    Physical page ids are a seeded permutation of the pool, so logical order
    and physical order never agree. Returns (page_table int32 [B, max_pages]
    filled with -1 past each sequence's pages, num_pages in the pool).
    """
    counts = [-(-int(t) // page_size) for t in tokens_per_seq]
    total = sum(counts)
    num_pages = total + spare
    perm = rng.permutation(num_pages).astype(np.int32)
    max_pages = max(counts) if counts else 0
    table = np.full((len(counts), max(max_pages, 1)), -1, dtype=np.int32)
    off = 0
    for b, c in enumerate(counts):
        table[b, :c] = perm[off : off + c]
        off += c
    return table, num_pages


def allocate_rings(rng: np.random.Generator, batch: int, spare: int = 2):
    """Seeded distinct ring ids for `batch` sequences; returns (ids int32 [B], num_rings)."""
    num_rings = batch + spare
    return rng.permutation(num_rings)[:batch].astype(np.int32), num_rings


@dataclass
class Structure:
    workload: str
    shape: HeadShape
    kinds: list
    hist: np.ndarray            # int32 [B] tokens already cached before the timed pass
    new: np.ndarray             # int32 [B] tokens processed by the pass
    page_table: np.ndarray      # int32 [B, max_pages]
    num_pages: int
    ring_id: np.ndarray         # int32 [B]
    num_rings: int
    extra: dict = field(default_factory=dict)

    @property
    def batch(self) -> int:
        return int(self.hist.shape[0])


def small_structure() -> Structure:
    rng = structure_rng("small")
    prefill, steps = 512, 16
    table, num_pages = allocate_pages(rng, [prefill + steps], spare=64 - 33)
    ring_id, num_rings = allocate_rings(rng, 1, spare=1)
    return Structure("small", SMALL_SHAPE, ["swa", "full"], np.array([0], np.int32),
                     np.array([prefill], np.int32), table, num_pages, ring_id, num_rings,
                     extra={"decode_steps": steps, "chunk": 128, "scale": 1.0 / 8.0})


def decode_structure() -> Structure:
    rng = structure_rng("decode")
    batch, hist = 64, 8192
    table, num_pages = allocate_pages(rng, [hist + 1] * batch)
    ring_id, num_rings = allocate_rings(rng, batch)
    return Structure("decode", BIG_SHAPE, GROUP_KINDS, np.full(batch, hist, np.int32),
                     np.ones(batch, np.int32), table, num_pages, ring_id, num_rings)


def chunked_structure() -> Structure:
    rng = structure_rng("chunked")
    batch, total, chunk = 4, 32768, 8192
    table, num_pages = allocate_pages(rng, [total] * batch)
    ring_id, num_rings = allocate_rings(rng, batch)
    return Structure("chunked", BIG_SHAPE, GROUP_KINDS, np.zeros(batch, np.int32),
                     np.full(batch, total, np.int32), table, num_pages, ring_id, num_rings,
                     extra={"chunk": chunk})


def reuse_structure() -> Structure:
    """Prefix-reuse batch. The reusable length L is NOT computed here: `hist`
    holds the cached prefix length P and extra['valid'] the SWA validity map
    of the last 2W cached positions; the caller applies the window-safe rule."""
    rng = structure_rng("reuse")
    batch = 32
    prefix = rng.integers(4096, 65536, size=batch, endpoint=True).astype(np.int32)
    frac = rng.uniform(0.0, 0.30, size=batch)
    suffix = rng.integers(512, 2048, size=batch, endpoint=True).astype(np.int32)
    evicted = []
    for b in range(batch):
        count = int(np.floor(frac[b] * WINDOW))
        offs = rng.choice(WINDOW, size=count, replace=False)
        evicted.append(np.sort(prefix[b] - WINDOW + offs).astype(np.int64))
    # token ids: the request repeats the cached prefix, then continues with new ids
    table, num_pages = allocate_pages(rng, (prefix + suffix).tolist())
    ring_id, num_rings = allocate_rings(rng, batch)
    return Structure("reuse", BIG_SHAPE, GROUP_KINDS, prefix, suffix, table, num_pages,
                     ring_id, num_rings, extra={"evicted": evicted, "frac": frac})


def reuse_tokens(struct: Structure, b: int):
    """Synthetic token ids for sequence b: (request tokens, cached tokens, swa_valid)."""
    rng = np.random.default_rng([WORKLOAD_IDS["reuse"], 1, b])
    p = int(struct.hist[b])
    s = int(struct.new[b])
    cached = rng.integers(0, 1 << 30, size=p, dtype=np.int64).astype(np.int32)
    request = np.concatenate([cached, rng.integers(1 << 30, 1 << 31, size=s, dtype=np.int64).astype(np.int32)])
    valid = np.ones(p, dtype=np.uint8)
    valid[struct.extra["evicted"][b]] = 0
    return request, cached, valid


def ragged_structure() -> Structure:
    rng = structure_rng("ragged")
    lens = np.concatenate([
        rng.integers(1 << 10, 1 << 16, size=12, endpoint=True),
        rng.integers(1 << 16, 1 << 18, size=8, endpoint=True),
        rng.integers(1 << 18, 1 << 20, size=4, endpoint=True),
    ]).astype(np.int32)
    table, num_pages = allocate_pages(rng, (lens + 1).tolist())
    ring_id, num_rings = allocate_rings(rng, len(lens))
    return Structure("ragged", BIG_SHAPE, GROUP_KINDS, lens, np.ones(len(lens), np.int32),
                     table, num_pages, ring_id, num_rings)


def value_generator(workload: str, layer: int, purpose: int, device):
    import torch

    g = torch.Generator(device=device)
    g.manual_seed(1000 * WORKLOAD_IDS[workload] + 10 * layer + purpose)
    return g


def normal_f32(shape, workload: str, layer: int, purpose: int, device):
    """float32 N(0,1) tensor from the seeded generator."""
    import torch

    return torch.randn(*shape, generator=value_generator(workload, layer, purpose, device),
                       device=device, dtype=torch.float32)


def normal_bf16(shape, workload: str, layer: int, purpose: int, device):
    """N(0,1) drawn in float32, rounded to bfloat16 (round-to-nearest-even)."""
    import torch

    return normal_f32(shape, workload, layer, purpose, device).to(torch.bfloat16)


# purposes
Q_VALUES, K_VALUES, V_VALUES = 0, 1, 2
