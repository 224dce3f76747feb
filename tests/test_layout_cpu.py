"""The tests' pool-layout decoders agree with the element formulas documented
in include/hybrid_attn.h (so GPU checks read the pools the way the ABI says)."""

import numpy as np
import pytest

from gpu_util import block_k, block_v


@pytest.mark.parametrize("d", [64, 128])
def test_block_decoders_match_documented_formula(d):
    rng = np.random.default_rng(0)
    vals = rng.standard_normal((16, d))
    k_enc = np.empty(16 * d)
    v_enc = np.empty(16 * d)
    for t in range(16):
        for ch in range(d):
            k_enc[((ch // 32) * 64 + ((ch % 32) // 8) * 16 + t) * 8 + ch % 8] = vals[t, ch]
            v_enc[((ch // 32) * 64 + (t // 4) * 16 + ch % 16) * 8 + ((ch % 32) // 16) * 4 + t % 4] = vals[t, ch]
    np.testing.assert_array_equal(block_k(k_enc[None], d)[0], vals)
    np.testing.assert_array_equal(block_v(v_enc[None], d)[0], vals)
