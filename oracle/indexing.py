"""Oracle: where each token's K/V lives in the two pools (test infrastructure only).

The pages split the KV cache into two physically separate pools
([YLY §2 "KVCache系统重构：让缓存真正省下来"], [HD12 "双池分治与三级缓存的工程实现"],
[HTX 工程二], [HD9 "三层 KVCache 系统"]):

* SWA pool: capacity fixed by the window, organised as a ring buffer with
  window-based eviction, storage O(W) per sequence and layer. Modelled here as
  W slots per sequence; the token at absolute position p lives in slot
  p mod W, so appending position p evicts position p - W.
* Full pool: grows on demand and is long-lived; the Full-attention index is
  the authoritative per-sequence index. Modelled as fixed-size pages and a
  per-sequence page table: position p lives in page page_table[p // P] at
  offset p mod P (P = page size, 16 tokens in every workload here).

Only the *logical* mapping is modelled (position -> slot, position -> page
and offset). The byte layout inside a slot or page belongs to the pool format
and is decoded by the tests.

Pins (tests/test_oracle_indexing.py): ring contents equal a
``collections.deque(maxlen=W)`` of the appended positions, and the closed form
"slot s holds the largest appended p with p = s (mod W)"; page locations
cover each (page, offset) exactly once for a permuted page table.
"""

from __future__ import annotations

import numpy as np


def ring_slot(pos, window: int):
    """Slot of absolute position `pos` in a W-slot ring (array or int)."""
    if window < 1:
        raise ValueError("window must be >= 1")
    return np.asarray(pos, dtype=np.int64) % window


def ring_contents(appended_positions, window: int) -> np.ndarray:
    """Position held by each of the W slots after appending positions in order.

    `appended_positions` must be strictly increasing (tokens are appended in
    sequence order). Slots never written hold -1.
    """
    pos = np.asarray(appended_positions, dtype=np.int64)
    if pos.size > 1 and np.any(np.diff(pos) <= 0):
        raise ValueError("appended positions must be strictly increasing")
    slots = np.full(window, -1, dtype=np.int64)
    for p in pos:
        slots[int(p) % window] = p
    return slots


def page_location(page_table_row, pos, page_size: int):
    """(physical page, offset within page) of absolute position(s) `pos`."""
    if page_size < 1:
        raise ValueError("page_size must be >= 1")
    pos = np.asarray(pos, dtype=np.int64)
    row = np.asarray(page_table_row, dtype=np.int64)
    logical_page = pos // page_size
    if np.any(logical_page >= row.shape[0]):
        raise ValueError("position beyond the sequence's page table")
    return row[logical_page], pos % page_size


def pages_needed(num_tokens: int, page_size: int) -> int:
    """Pages a sequence of `num_tokens` tokens occupies in the Full pool."""
    return -(-int(num_tokens) // page_size)
