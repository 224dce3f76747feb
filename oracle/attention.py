"""Oracle: masked softmax attention in float64 (test infrastructure only).

What it computes
----------------
The pages describe a 70-layer model in which most layers attend only to the
most recent 128 tokens (sliding-window attention, SWA) and one layer in seven
attends to the whole history (full causal attention) -- [HTX 工程一],
[YLY §1 为什么选择 Hybrid SWA 架构], [HD9 "Hybrid SWA：用 1/7 计算量捕获长程依赖"].
The dual-pool KV cache changes only where K/V are stored, not what attention
computes, so the oracle is plain attention over *logically gathered* K/V:
arrays indexed by absolute token position 0..T-1.

For query position t, query head h, kv head g(h) = h // (Hq // Hkv)
(contiguous GQA groups; the pages never mention GQA, this is the usual
convention), scale s = 1/sqrt(D) unless given:

    visible(t) = { j : lo(t) <= j <= t },
        lo(t) = max(0, t - W + 1)   for SWA   (W keys including the query itself)
        lo(t) = 0                   for FULL
    score_j = s * <q_{t,h}, k_{j,g}>              (j visible, else -inf)
    lse     = m + ln sum_j exp(score_j - m),      m = max_j score_j
    o       = sum_j exp(score_j - lse) * v_{j,g}

The window reading (W keys *including* the query's own token) is the plainest
reading of the pages' statement that SWA layers see only the latest 128 tokens,
and it is the one under which a W-slot ring buffer holds a decode query's
whole window.

Pins (tests/test_oracle_attention.py): all-equal-keys closed form (window
bounds, scale, log base), W = 1 closed form, SWA == FULL when W >= T,
torch.nn.functional.scaled_dot_product_attention in float64 with an explicit
boolean mask and repeated KV heads, scipy.special.logsumexp for LSE, GQA ==
MHA with repeated KV heads, and a scalar pure-Python brute force on tiny
inputs (written in the test, not here).
"""

from __future__ import annotations

import numpy as np

SWA = "swa"
FULL = "full"


def visible_mask(q_pos: np.ndarray, num_keys: int, kind: str, window: int) -> np.ndarray:
    """Boolean mask M[i, j] = key position j is visible to query position q_pos[i]."""
    if kind not in (SWA, FULL):
        raise ValueError(f"kind must be 'swa' or 'full', got {kind!r}")
    t = np.asarray(q_pos, dtype=np.int64)[:, None]
    j = np.arange(num_keys, dtype=np.int64)[None, :]
    mask = j <= t
    if kind == SWA:
        if window < 1:
            raise ValueError("window must be >= 1")
        mask &= j >= t - window + 1
    return mask


def attend(q, k, v, q_pos, kind: str, window: int, scale: float | None = None):
    """Attention rows of one sequence.

    q      [n, Hq, D]   queries at absolute positions q_pos[n]
    k, v   [T, Hkv, D]  logical K/V of the sequence, row j = position j
                        (any float dtype; converted to float64 exactly)
    q_pos  [n]          int positions, each < T
    kind   'swa' | 'full'
    window W (used for 'swa')
    Returns (o [n, Hq, D] float64, lse [n, Hq] float64).
    """
    q = np.asarray(q)
    n, hq, d = q.shape
    t_keys, hkv, d2 = k.shape
    if d2 != d or v.shape != k.shape:
        raise ValueError("q/k/v head_dim or k/v shapes disagree")
    if hq % hkv != 0:
        raise ValueError("num_q_heads must be a multiple of num_kv_heads")
    q_pos = np.asarray(q_pos, dtype=np.int64)
    if q_pos.shape != (n,):
        raise ValueError("q_pos must have one position per query row")
    if n and (q_pos.min() < 0 or q_pos.max() >= t_keys):
        raise ValueError("query position outside the key range")
    if scale is None:
        scale = 1.0 / np.sqrt(d)
    group = hq // hkv

    # Keys beyond the last query position are never visible; dropping them
    # removes only exact-zero terms.
    last = int(q_pos.max()) + 1 if n else 0
    mask = visible_mask(q_pos, last, kind, window)
    out = np.zeros((n, hq, d), dtype=np.float64)
    lse = np.zeros((n, hq), dtype=np.float64)
    for g in range(hkv):
        kg = np.asarray(k[:last, g, :], dtype=np.float64)
        vg = np.asarray(v[:last, g, :], dtype=np.float64)
        for h in range(g * group, (g + 1) * group):
            qh = np.asarray(q[:, h, :], dtype=np.float64)
            s = scale * (qh @ kg.T)                       # [n, last]
            s = np.where(mask, s, -np.inf)
            m = s.max(axis=1, keepdims=True)              # finite: each row sees itself
            lse_h = m[:, 0] + np.log(np.exp(s - m).sum(axis=1))
            p = np.exp(s - lse_h[:, None])
            out[:, h, :] = p @ vg
            lse[:, h] = lse_h
    return out, lse

