"""Pins of the oracle's quantizers: an exact rational re-derivation of the
group rule on small inputs, the max-abs invariant, metamorphic relations,
the per-element error bound, layout identities and edge cases."""

import math
from fractions import Fraction

import numpy as np
import pytest

from oracle import e4m3, quant
import synth

from test_oracle_codec import brute_encode


# ----------------------------------------------------------- exact re-derivation
def f32_round(fr):
    """Fraction -> nearest float32 (ties to even), exactly, by search over
    the float32 neighbours of a float64 approximation."""
    approx = np.float32(float(fr))
    cands = {approx, np.nextafter(approx, np.float32(np.inf)),
             np.nextafter(approx, np.float32(-np.inf))}
    best = None
    for c in sorted(cands, key=float):
        d = abs(Fraction(float(c)) - fr)
        even = (np.array(c, np.float32).view(np.uint32) & 1) == 0
        if best is None or d < best[0] or (d == best[0] and even):
            best = (d, c)
    return np.float32(best[1])


def exact_group(xs):
    """The group rule of the pages (max-abs mapped to 448) with every FP32
    operation rounded exactly from rationals: returns (codes, s)."""
    amax = max((abs(Fraction(float(v))) for v in xs), default=Fraction(0))
    amax = max(amax, Fraction(2) ** -100)
    s = f32_round(amax / 448)
    inv = f32_round(Fraction(448) / amax)
    codes = [brute_encode(f32_round(Fraction(float(v)) * Fraction(float(inv)))
                          if float(v) != 0 or math.copysign(1, float(v)) > 0
                          else float(v))
             for v in xs]
    return codes, s


def _bf16_values(a):
    return synth.to_bf16(a).float().numpy()


def test_act_matches_exact_rederivation():
    x = _bf16_values(synth.general(48, 300, seed=21, outlier_frac=0.02, outlier_mul=60.0))
    x[2, 128:256] = 0.0                    # a zero group
    x[3, :5] = -0.0
    x[4, 256:] *= 1e-30                    # a tiny trailing partial group
    q, s = quant.quant_act_1x128(x)
    for r in range(x.shape[0]):
        for j in range(3):
            codes, sj = exact_group(x[r, 128 * j:128 * (j + 1)])
            assert s[r, j] == sj, (r, j)
            assert q[r, 128 * j:128 * (j + 1)].tolist() == codes, (r, j)


def test_weight_block_matches_exact_rederivation():
    w = synth.general(130, 140, seed=22).astype(np.float32) * np.float32(0.02)
    q, s, q_t = quant.quant_weight_128x128(w)
    assert s.shape == (2, 2)
    for i in range(2):
        for j in range(2):
            blk = w[128 * i:128 * (i + 1), 128 * j:128 * (j + 1)]
            codes, sij = exact_group(blk.reshape(-1))
            assert s[i, j] == sij
            assert q[128 * i:128 * (i + 1), 128 * j:128 * (j + 1)].reshape(-1).tolist() == codes


# -------------------------------------------------------------------- invariants
def _groups_act(x, q):
    for r in range(x.shape[0]):
        for j in range(0, x.shape[1], 128):
            yield x[r, j:j + 128], q[r, j:j + 128]


@pytest.mark.parametrize("seed", [1, 2, 3])
def test_max_abs_element_encodes_to_448(seed):
    x = _bf16_values(synth.general(64, 1000, seed=seed, kind="t3"))
    q, s = quant.quant_act_1x128(x)
    for xv, qv in _groups_act(x, q):
        amax = np.abs(xv).max()
        hit = np.abs(xv) == amax
        assert np.all((qv[hit] & 0x7F) == 0x7E)
        assert np.all((qv[~hit] & 0x7F) <= 0x7E)


def test_scaling_by_powers_of_two_is_exact():
    x = _bf16_values(synth.general(8, 384, seed=5))
    q, s = quant.quant_act_1x128(x)
    for j in (-20, -3, 1, 7, 30):
        q2, s2 = quant.quant_act_1x128(x * np.float32(2.0 ** j))
        assert np.array_equal(q2, q)
        assert np.array_equal(s2, s * np.float32(2.0 ** j))


def test_negation_flips_sign_bits_only():
    x = _bf16_values(synth.general(8, 384, seed=6))
    q, s = quant.quant_act_1x128(x)
    qn, sn = quant.quant_act_1x128(-x)
    assert np.array_equal(qn, q ^ 0x80) and np.array_equal(sn, s)


def test_permutation_within_group_permutes_codes():
    x = _bf16_values(synth.general(4, 256, seed=8))
    q, s = quant.quant_act_1x128(x)
    perm = np.random.Generator(np.random.PCG64(9)).permutation(128)
    xp = x.copy()
    xp[:, 128:] = x[:, 128:][:, perm]
    qp, sp = quant.quant_act_1x128(xp)
    assert np.array_equal(sp, s)
    assert np.array_equal(qp[:, 128:], q[:, 128:][:, perm])
    assert np.array_equal(qp[:, :128], q[:, :128])


def test_error_bound():
    x = _bf16_values(synth.general(32, 1024, seed=10, outlier_frac=0.01, outlier_mul=100.0))
    q, s = quant.quant_act_1x128(x)
    deq = e4m3.decode(q) * s.astype(np.float64)[:, np.arange(1024) // 128]
    sfull = s.astype(np.float64)[:, np.arange(1024) // 128]
    y = np.abs(x.astype(np.float64)) / sfull            # magnitude on the E4M3 grid
    err = np.abs(deq - x)
    normal = y >= 2.0 ** -6 * (1 + 2.0 ** -20)
    slack = 1 + 2.0 ** -18
    assert np.all(err[normal] <= 2.0 ** -4 * np.abs(x[normal]) * slack)
    assert np.all(err[~normal] <= 2.0 ** -10 * sfull[~normal] * slack)


# ----------------------------------------------------------------------- layouts
def test_weight_transposed_codes_are_the_transpose():
    w = synth.general(300, 260, seed=12).astype(np.float32)
    q, s, q_t = quant.quant_weight_128x128(w)
    assert q_t.shape == (260, 300) and np.array_equal(q_t, q.T)
    # a block's scale does not change when the matrix is transposed
    qT, sT, _ = quant.quant_weight_128x128(np.ascontiguousarray(w.T))
    assert np.array_equal(sT, s.T) and np.array_equal(qT, q.T)


@pytest.mark.parametrize("shape", [(128, 128), (300, 70), (1, 5), (257, 129)])
def test_transpose_equals_act_of_transposed_input(shape):
    x = _bf16_values(synth.general(*shape, seed=13, kind="t3"))
    q_t, s_t = quant.quant_transpose(x)
    q2, s2 = quant.quant_act_1x128(np.ascontiguousarray(x.T))
    assert np.array_equal(q_t, q2) and np.array_equal(s_t, s2)


# -------------------------------------------------------------------- edge cases
def test_zero_and_signed_zero_groups():
    x = np.zeros((2, 256), np.float32)
    x[1, :] = -0.0
    q, s = quant.quant_act_1x128(x)
    assert np.all(q[0] == 0) and np.all(q[1] == 0x80)
    assert np.all(s == np.float32(2.0 ** -100) / np.float32(448.0))


def test_partial_groups_and_empty_inputs():
    x = _bf16_values(synth.general(3, 130, seed=14))
    q, s = quant.quant_act_1x128(x)
    assert s.shape == (3, 2)
    for r in range(3):
        tail = x[r, 128:]
        assert s[r, 1] == np.float32(np.abs(tail).max()) / np.float32(448.0)
    for shape in [(0, 256), (5, 0), (0, 0)]:
        q, s = quant.quant_act_1x128(np.zeros(shape, np.float32))
        assert q.shape == shape and s.shape == (shape[0], (shape[1] + 127) // 128)
        qt, st = quant.quant_transpose(np.zeros(shape, np.float32))
        assert qt.shape == shape[::-1] and st.shape == (shape[1], (shape[0] + 127) // 128)
        qw, sw, qwt = quant.quant_weight_128x128(np.zeros(shape, np.float32))
        assert qw.shape == shape and qwt.shape == shape[::-1]
