"""Oracle: "window-safe length" prefix matching, by brute force (test infrastructure only).

Under SWA, equal token prefixes no longer imply that the cached K/V are
still there: the SWA slots of a cached prefix may have been evicted, and a
match that trusts token equality alone ("false hit") reads invalid or
overwritten K/V ([HTX 工程三], [YLY §2 "KVCache系统重构：让缓存真正省下来"],
[HD9 "Hybrid SWA：用 1/7 计算量捕获长程依赖"]). The pages' fix is the
window-safe length: a cached prefix is reusable only up to a length L whose
last W tokens still have valid SWA slots, i.e. the match is clipped back to a
window boundary ([YLY, same section], [HD12 "双池分治与三级缓存的工程实现"]).
[HD12 "边缘部署的工程权衡与参数清单"] notes that the rule is tied to W.

Reading used (plainest one the pages support):
    m = LCP(request tokens, cached tokens)
    L = max { L <= m : every position in [max(0, L - W), L) has a valid SWA slot }
The Full pool is authoritative and long-lived, so it is taken as valid over
the whole cached prefix; L = 0 is always safe (empty range). Under the
W-keys-including-self window only W-1 tail slots are strictly needed; the
rule is implemented as the pages state it (W slots).

Pins (tests/test_oracle_window_safe.py): hand-worked cases in
tests/golden/window_safe_cases.json (each citing the rule above) and
structural invariants over exhaustive tiny inputs.
"""

from __future__ import annotations


def common_prefix_length(a, b) -> int:
    """Length of the longest common prefix of two token sequences."""
    n = min(len(a), len(b))
    i = 0
    while i < n and int(a[i]) == int(b[i]):
        i += 1
    return i


def window_safe_length(request_tokens, cached_tokens, swa_valid, window: int) -> int:
    """Largest reusable prefix length under the window-safe rule (brute force).

    request_tokens  tokens of the new request
    cached_tokens   tokens of the cached prefix
    swa_valid       one flag per cached position: its SWA slot is still valid
    window          W
    """
    if window < 1:
        raise ValueError("window must be >= 1")
    if len(swa_valid) != len(cached_tokens):
        raise ValueError("one validity flag per cached token is required")
    m = common_prefix_length(request_tokens, cached_tokens)
    for length in range(m, -1, -1):
        lo = max(0, length - window)
        if all(bool(swa_valid[j]) for j in range(lo, length)):
            return length
    return 0  # unreachable: length 0 has an empty tail
