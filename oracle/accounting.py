"""Oracle: visible-pair and KV-size counts behind the pages' 1/7 figures
(test infrastructure only).

The pages state that with 60 of 70 layers using a 128-token window and 10
layers attending to everything, the KV cache shrinks to about 1/7 of an
all-full-attention model and prefill attention compute shrinks about as much
([HTX 工程一], [YLY §1 "为什么选择 Hybrid SWA 架构"],
[HD12 "架构层面的 KV Cache 压缩"]); the layers are interleaved 6:1
([HD9 "Hybrid SWA：用 1/7 计算量捕获长程依赖"], [HD9 "生产级调参清单"]).

These counts follow directly from the visibility rule of oracle.attention:
a query at position t sees min(t+1, W) keys in an SWA layer and t+1 keys in
a full layer; a sequence of N tokens keeps min(N, W) K/V rows per SWA layer
and N per full layer.

Pins (tests/test_oracle_accounting.py): brute-force counts of
oracle.attention.visible_mask, and the pages' printed figures
(tests/golden/pages_figures.json): 70 layers = 60 SWA + 10 full, W = 128,
ratios tending to 1/7.
"""

from __future__ import annotations


def visible_keys(t: int, kind: str, window: int) -> int:
    """Number of keys a query at position t attends to."""
    if kind == "swa":
        return min(t + 1, window)
    if kind == "full":
        return t + 1
    raise ValueError(kind)


def visible_pairs(hist: int, n_new: int, kind: str, window: int) -> int:
    """Sum of visible keys over queries at positions hist .. hist+n_new-1."""
    return sum(visible_keys(t, kind, window) for t in range(hist, hist + n_new))


def kv_rows(num_tokens: int, kind: str, window: int) -> int:
    """K/V rows one layer must keep for a sequence of num_tokens tokens."""
    if kind == "swa":
        return min(num_tokens, window)
    if kind == "full":
        return num_tokens
    raise ValueError(kind)


def hybrid_kv_ratio(num_tokens: int, n_swa: int, n_full: int, window: int) -> float:
    """KV size of the hybrid stack divided by an all-full stack of the same depth."""
    hybrid = n_swa * kv_rows(num_tokens, "swa", window) + n_full * kv_rows(num_tokens, "full", window)
    return hybrid / ((n_swa + n_full) * num_tokens)


def hybrid_prefill_pair_ratio(num_tokens: int, n_swa: int, n_full: int, window: int) -> float:
    """Attention (query, key) pairs of a full prefill, hybrid over all-full."""
    swa = visible_pairs(0, num_tokens, "swa", window)
    full = visible_pairs(0, num_tokens, "full", window)
    return (n_swa * swa + n_full * full) / ((n_swa + n_full) * full)
