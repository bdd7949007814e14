"""Pins of the oracle's microscaling (MXFP8 E4M3) variant.

* E8M0 scale: closed form floor(log2 amax) - 8 + 127 on exact powers of two
  and their neighbours, the all-zero block, the clamp.
* Codes: a brute-force nearest-grid search in rationals on x / X for every
  element of small random blocks (including blocks whose largest element
  saturates), the max-abs invariant (the block's largest element encodes to
  a magnitude in [256, 448]), power-of-two and sign metamorphic relations.
* GEMM: operands built so that quantization is exact (every 32-block's
  max-abs is in [256, 448] * 2^e with grid values), so the product must equal
  the integer matmul of the constructed matrices.
"""

from fractions import Fraction

import numpy as np
import pytest

from oracle import e4m3, mx

from test_oracle_codec import brute_encode

GRID = np.array(sorted({abs(v) for v in e4m3.decode(e4m3.finite_codes()) if abs(v) <= 448}))


def test_e8m0_closed_form():
    for k in range(-120, 120, 7):
        for m in (1.0, 1.5, 1.999999):
            amax = m * 2.0 ** k
            want = min(max(k - 8 + 127, 0), 254)
            assert mx.e8m0_of_amax(np.array([amax]))[0] == want, (k, m)
    assert mx.e8m0_of_amax(np.array([0.0]))[0] == 0
    assert mx.e8m0_of_amax(np.array([2.0 ** -140]))[0] == 0          # clamped below
    assert mx.scale_value(np.array([127]))[0] == 1.0


@pytest.mark.parametrize("seed", range(4))
def test_codes_match_brute_force(seed):
    rng = np.random.Generator(np.random.PCG64(seed))
    x = (rng.standard_t(3, size=(8, 96)) * rng.choice([1e-3, 1.0, 300.0], size=(8, 1))).astype(np.float32)
    x[0, 5] = 0.0
    x[1, :32] = 0.0                                     # an all-zero block
    x[2, 40] = -x[2, 32:64].__abs__().max() * 1.0       # a negative block maximum
    q, s = mx.quant_mx(x)
    for r in range(x.shape[0]):
        for c in range(x.shape[1]):
            X = Fraction(2) ** (int(s[r, c // 32]) - 127)
            y = np.float32(Fraction(float(x[r, c])) / X)
            assert q[r, c] == brute_encode(y), (r, c)


def test_block_maximum_lands_in_the_top_binade():
    rng = np.random.Generator(np.random.PCG64(11))
    x = (rng.standard_normal((64, 256)) * np.exp(rng.uniform(-20, 20, size=(64, 1)))).astype(np.float32)
    q, s = mx.quant_mx(x)
    dq = np.abs(e4m3.decode(q)).reshape(64, 8, 32)
    top = dq.max(axis=2)
    assert np.all((top >= 256) & (top <= 448))


def test_power_of_two_and_sign_relations():
    rng = np.random.Generator(np.random.PCG64(12))
    x = rng.standard_normal((16, 128)).astype(np.float32)
    q, s = mx.quant_mx(x)
    for j in (-5, 3, 20):
        q2, s2 = mx.quant_mx(x * np.float32(2.0 ** j))
        assert np.array_equal(q, q2) and np.array_equal(s2.astype(int), s.astype(int) + j)
    qn, sn = mx.quant_mx(-x)
    assert np.array_equal(qn, q ^ 0x80) and np.array_equal(sn, s)


def _exact_mx_matrix(rows, cols, rng):
    """Grid values whose every 32-block has max-abs in [256, 448], times a
    random power of two per block: MX quantization is exact on it.  Returns
    (float32 matrix, its integer multiple by 2^40)."""
    v = rng.choice(GRID[GRID <= 448], size=(rows, cols)) * rng.choice([-1.0, 1.0], size=(rows, cols))
    for r in range(rows):
        for b in range(0, cols, 32):
            v[r, b + int(rng.integers(32))] = rng.choice([256.0, 288.0, 448.0])
            v[r, b:b + 32] *= 2.0 ** int(rng.integers(-12, 12))
    ints = np.rint(v * 2.0 ** 40).astype(object)
    return v.astype(np.float32), ints


def test_gemm_closed_form():
    rng = np.random.Generator(np.random.PCG64(13))
    a, ai = _exact_mx_matrix(6, 128, rng)
    b, bi = _exact_mx_matrix(5, 128, rng)
    aq, as_ = mx.quant_mx(a)
    bq, bs = mx.quant_mx(b)
    assert np.array_equal(mx.dequant_mx(aq, as_), a.astype(np.float64))
    y, s = mx.gemm_mx_ref(aq, as_, bq, bs)
    exact = ai.dot(bi.T)
    for m in range(6):
        for n in range(5):
            want = Fraction(int(exact[m, n]), 2 ** 80)
            assert abs(Fraction(float(y[m, n])) - want) <= Fraction(130) * Fraction(2) ** -53 * Fraction(float(s[m, n]))
