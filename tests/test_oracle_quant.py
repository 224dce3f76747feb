"""Pins of the INT8 KV quantization oracle (oracle/quant.py) to its
definition: exact arithmetic with fractions, the closed-form properties of
symmetric absmax scaling, ties to even, and the bf16 input rounding."""

from fractions import Fraction

import numpy as np

from oracle.quant import bf16_round, dequantize_rows, quantize_rows


def f32_nearest(fr: Fraction) -> np.float32:
    """The float32 nearest to an exact rational (ties to even), by search."""
    f = np.float32(float(fr))          # within one ulp
    best = None
    for cand in (np.nextafter(f, np.float32(-np.inf)), f, np.nextafter(f, np.float32(np.inf))):
        err = abs(Fraction(float(cand)) - fr)
        key = (err, int(np.float32(cand).view(np.uint32)) & 1)
        if best is None or key < best[0]:
            best = (key, cand)
    return np.float32(best[1])


def test_codes_and_scales_follow_exact_arithmetic():
    rng = np.random.default_rng(0)
    x = bf16_round(rng.standard_normal((40, 64)).astype(np.float32) * 3)
    codes, scale = quantize_rows(x)
    for r in range(x.shape[0]):
        amax = max(abs(Fraction(float(v))) for v in x[r])
        s = f32_nearest(amax / 127)
        assert scale[r] == s
        for d in range(x.shape[1]):
            ratio = f32_nearest(Fraction(float(x[r, d])) / Fraction(float(s)))
            q = Fraction(float(ratio))
            fl = q.numerator // q.denominator
            frac = q - fl
            exp = fl + (1 if frac > Fraction(1, 2) or (frac == Fraction(1, 2) and fl % 2) else 0)
            assert codes[r, d] == max(-127, min(127, exp))


def test_absmax_properties():
    rng = np.random.default_rng(1)
    x = bf16_round(rng.standard_normal((200, 128)).astype(np.float32))
    codes, scale = quantize_rows(x)
    arg = np.argmax(np.abs(x), axis=1)
    rows = np.arange(x.shape[0])
    assert np.all(np.abs(codes[rows, arg]) == 127)                          # the absmax element saturates
    assert np.all(np.sign(codes[rows, arg]) == np.sign(x[rows, arg]))
    err = np.abs(dequantize_rows(codes, scale) - x)
    # half a step, plus the float32 rounding of x / scale (at most 127 * 2^-24 of a step)
    assert np.all(err <= scale[:, None] * (0.5 + 127 * 2.0 ** -24))
    assert np.all(np.abs(codes) <= 127)
    neg_codes, neg_scale = quantize_rows(-x)                                # odd symmetry
    assert np.array_equal(neg_codes, -codes) and np.array_equal(neg_scale, scale)


def test_zero_rows_grid_rows_and_ties():
    codes, scale = quantize_rows(np.zeros((2, 8), np.float32))
    assert np.all(codes == 0) and np.all(scale == 0)
    # a row already on a grid whose step is exact in float32 comes back unchanged
    step = np.float32(2.0 ** -3)
    q = np.array([[127, -127, 0, 5, -6, 64, 1, -1]], np.float32)
    codes, scale = quantize_rows(q * step)
    assert scale[0] == step
    assert codes.tolist() == q.astype(np.int8).tolist()
    # ties go to even: amax 127 gives scale 1, so x = k + 0.5 is an exact tie
    x = np.array([[127, 0.5, 1.5, 2.5, -0.5, -1.5, -2.5, 3.5]], np.float32)
    codes, scale = quantize_rows(x)
    assert scale[0] == 1.0
    assert codes.tolist() == [[127, 0, 2, 2, 0, -2, -2, 4]]


def test_bf16_rounding():
    x = np.array([1.0, 1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, -1.0 - 2 ** -8, 1.0 + 2 ** -7 + 2 ** -9], np.float32)
    # halfway cases go to even mantissas; above halfway rounds up
    assert bf16_round(x).tolist() == [1.0, 1.0, 1.0 + 2 ** -6, -1.0, 1.0 + 2 ** -7]
