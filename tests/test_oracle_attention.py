"""Pins for oracle.attention against things other than itself.

Each test is chosen so a plausible slip in the oracle fails it:
* window off-by-one, missing scale, wrong log base   -> all-equal-keys closed form, W = 1
* transposed operand / wrong mask orientation          -> torch SDPA with explicit mask
* wrong GQA head mapping                               -> SDPA with repeat_interleave, GQA == MHA
* wrong LSE                                            -> closed forms, scipy logsumexp
"""

import math

import numpy as np
import pytest
import torch
from scipy.special import logsumexp

from oracle.attention import FULL, SWA, attend, visible_mask


def _rand(rng, *shape):
    return rng.standard_normal(shape)


@pytest.mark.parametrize("kind,window", [(SWA, 3), (SWA, 4), (SWA, 8), (FULL, 4)])
def test_all_equal_keys_closed_form(kind, window):
    # With every key equal, each visible score equals s*<q,k>: the softmax is
    # uniform over the visible set, so lse = s*<q,k> + ln|visible| and o is the
    # plain mean of the visible values. |visible| = min(t+1, W) for SWA.
    rng = np.random.default_rng(1)
    T, hq, hkv, d = 11, 4, 2, 8
    kvec = _rand(rng, hkv, d)
    k = np.broadcast_to(kvec, (T, hkv, d)).copy()
    v = _rand(rng, T, hkv, d)
    q = _rand(rng, T, hq, d)
    pos = np.arange(T)
    o, lse = attend(q, k, v, pos, kind, window, scale=0.3)
    for t in range(T):
        lo = max(0, t - window + 1) if kind == SWA else 0
        count = t - lo + 1
        for h in range(hq):
            g = h // (hq // hkv)
            assert lse[t, h] == pytest.approx(0.3 * float(q[t, h] @ kvec[g]) + math.log(count), abs=1e-12)
            np.testing.assert_allclose(o[t, h], v[lo : t + 1, g].mean(axis=0), atol=1e-12)


def test_window_one_is_self_only():
    rng = np.random.default_rng(2)
    T, hq, hkv, d = 9, 2, 1, 4
    q, k, v = _rand(rng, T, hq, d), _rand(rng, T, hkv, d), _rand(rng, T, hkv, d)
    o, lse = attend(q, k, v, np.arange(T), SWA, 1)
    for h in range(hq):
        np.testing.assert_allclose(o[:, h], v[:, 0], atol=1e-14)
        np.testing.assert_allclose(lse[:, h], (q[:, h] * k[:, 0]).sum(-1) / 2.0, atol=1e-12)


@pytest.mark.parametrize("window", [16, 17, 100])
def test_swa_equals_full_when_window_covers_sequence(window):
    rng = np.random.default_rng(3)
    T = 16
    q, k, v = _rand(rng, T, 4, 8), _rand(rng, T, 1, 8), _rand(rng, T, 1, 8)
    o_s, l_s = attend(q, k, v, np.arange(T), SWA, window)
    o_f, l_f = attend(q, k, v, np.arange(T), FULL, window)
    np.testing.assert_array_equal(o_s, o_f)
    np.testing.assert_array_equal(l_s, l_f)


def test_window_changes_result_when_shorter():
    # Guard against a mask that ignores W entirely.
    rng = np.random.default_rng(4)
    T = 12
    q, k, v = _rand(rng, T, 2, 8), _rand(rng, T, 1, 8), _rand(rng, T, 1, 8)
    o_s, _ = attend(q, k, v, np.arange(T), SWA, 4)
    o_f, _ = attend(q, k, v, np.arange(T), FULL, 4)
    np.testing.assert_array_equal(o_s[:4], o_f[:4])
    assert np.abs(o_s[4:] - o_f[4:]).max() > 1e-3


@pytest.mark.parametrize("kind,window", [(FULL, 0), (SWA, 1), (SWA, 5), (SWA, 32)])
@pytest.mark.parametrize("hq,hkv", [(4, 1), (8, 2), (6, 6)])
def test_matches_torch_sdpa(kind, window, hq, hkv):
    rng = np.random.default_rng(5)
    T, d = 40, 16
    q, k, v = _rand(rng, T, hq, d), _rand(rng, T, hkv, d), _rand(rng, T, hkv, d)
    scale = 0.21
    o, lse = attend(q, k, v, np.arange(T), kind, window, scale=scale)

    g = hq // hkv
    qt = torch.from_numpy(q).permute(1, 0, 2)                       # [Hq, T, D]
    kt = torch.from_numpy(k).permute(1, 0, 2).repeat_interleave(g, 0)
    vt = torch.from_numpy(v).permute(1, 0, 2).repeat_interleave(g, 0)
    i = torch.arange(T)[:, None]
    j = torch.arange(T)[None, :]
    allowed = j <= i
    if kind == SWA:
        allowed &= j > i - window
    ref = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, attn_mask=allowed, scale=scale)
    np.testing.assert_allclose(o, ref.permute(1, 0, 2).numpy(), atol=1e-12)

    scores = scale * torch.matmul(qt, kt.transpose(1, 2)).numpy()
    scores = np.where(allowed.numpy()[None], scores, -np.inf)
    np.testing.assert_allclose(lse, logsumexp(scores, axis=-1).T, atol=1e-12)


def test_gqa_equals_mha_with_repeated_kv():
    rng = np.random.default_rng(6)
    T, hq, hkv, d = 20, 8, 2, 8
    q, k, v = _rand(rng, T, hq, d), _rand(rng, T, hkv, d), _rand(rng, T, hkv, d)
    o1, l1 = attend(q, k, v, np.arange(T), SWA, 6)
    o2, l2 = attend(q, np.repeat(k, 4, axis=1), np.repeat(v, 4, axis=1), np.arange(T), SWA, 6)
    np.testing.assert_array_equal(o1, o2)
    np.testing.assert_array_equal(l1, l2)


def _bruteforce(q, k, v, q_pos, kind, window, scale):
    hq, hkv, d = q.shape[1], k.shape[1], q.shape[2]
    out = np.zeros(q.shape)
    lse = np.zeros(q.shape[:2])
    for i, t in enumerate(q_pos):
        lo = max(0, t - window + 1) if kind == SWA else 0
        for h in range(hq):
            g = h // (hq // hkv)
            sc = [scale * sum(float(q[i, h, c]) * float(k[j, g, c]) for c in range(d)) for j in range(lo, t + 1)]
            mx = max(sc)
            ls = mx + math.log(sum(math.exp(x - mx) for x in sc))
            lse[i, h] = ls
            for c in range(d):
                out[i, h, c] = sum(math.exp(sc[jj] - ls) * float(v[lo + jj, g, c]) for jj in range(len(sc)))
    return out, lse


@pytest.mark.parametrize("kind,window", [(SWA, 3), (FULL, 0)])
def test_scalar_bruteforce_tiny(kind, window):
    rng = np.random.default_rng(7)
    T, hq, hkv, d = 7, 4, 2, 3
    q, k, v = _rand(rng, T, hq, d), _rand(rng, T, hkv, d), _rand(rng, T, hkv, d)
    pos = np.array([0, 2, 3, 6])
    o, lse = attend(q[pos], k, v, pos, kind, window, scale=0.7)
    ob, lb = _bruteforce(q[pos], k, v, pos, kind, window, 0.7)
    np.testing.assert_allclose(o, ob, atol=1e-12)
    np.testing.assert_allclose(lse, lb, atol=1e-12)


def test_single_row_equals_row_of_full_prefill():
    # Decode of the token at position t sees exactly what prefill row t sees.
    rng = np.random.default_rng(8)
    T = 30
    q, k, v = _rand(rng, T, 4, 8), _rand(rng, T, 1, 8), _rand(rng, T, 1, 8)
    o_all, l_all = attend(q, k, v, np.arange(T), SWA, 7)
    for t in (0, 6, 7, 29):
        o1, l1 = attend(q[t : t + 1], k[: t + 1], v[: t + 1], [t], SWA, 7)
        np.testing.assert_allclose(o1[0], o_all[t], atol=1e-13)
        np.testing.assert_allclose(l1[0], l_all[t], atol=1e-13)


def test_visible_mask_counts():
    m = visible_mask(np.arange(10), 10, SWA, 4)
    assert m.sum(axis=1).tolist() == [1, 2, 3, 4, 4, 4, 4, 4, 4, 4]
    assert visible_mask(np.arange(5), 5, FULL, 0).sum() == 15


def test_rejects_bad_arguments():
    z = np.zeros((2, 4, 8))
    kv = np.zeros((2, 3, 8))
    with pytest.raises(ValueError):
        attend(z, kv, kv, [0, 1], SWA, 4)          # Hq not a multiple of Hkv
    with pytest.raises(ValueError):
        attend(z, np.zeros((2, 1, 8)), np.zeros((2, 1, 8)), [0, 2], FULL, 4)
    with pytest.raises(ValueError):
        attend(z, np.zeros((2, 1, 8)), np.zeros((2, 1, 8)), [0, 1], "local", 4)
