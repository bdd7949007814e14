"""Pins of the oracle's grouped (MoE) backward references.

* Layout: for many random expert offsets (empty experts, multiples of 128,
  single tokens) the padded chunk ranges never overlap and stay inside the
  capacity; padding columns are code 0.
* Quantizer: every (channel, expert, 128-token group) is re-derived with exact
  rational arithmetic from the expert's own tokens only, so a group that
  leaked into the next expert, or a scale taken over padding, fails.
* Aligned experts (offsets multiples of 128) reduce to the plain pinned
  quant_transpose, and the sum of their weight gradients to the dense one.
* GEMMs: closed forms built so that quantization is exact (every group's
  max-abs is 448 * 2^e), and exact rationals on sampled outputs.
"""

from fractions import Fraction

import numpy as np
import pytest

import oracle
from oracle import e4m3
import synth

from test_oracle_gemm import pow2_matrix, _close_to_exact
from test_oracle_quant import exact_group


def _offsets(counts):
    return np.concatenate([[0], np.cumsum(counts)]).astype(np.int64)


RAGGED = [5, 0, 295, 1, 399, 128, 0, 130]


def test_padded_layout_never_overlaps():
    rng = np.random.Generator(np.random.PCG64(11))
    for trial in range(400):
        e = int(rng.integers(1, 12))
        kind = trial % 4
        if kind == 0:
            counts = rng.integers(0, 400, size=e)
        elif kind == 1:
            counts = 128 * rng.integers(0, 4, size=e)
        elif kind == 2:
            counts = rng.choice([0, 1, 127, 128, 129, 255, 256, 257], size=e)
        else:
            counts = rng.integers(0, 3, size=e)
        off = _offsets(counts)
        p = oracle.padded_starts(off)
        cap = oracle.token_capacity(off[-1], e)
        assert cap % 128 == 0 and np.all(p % 128 == 0)
        end = 0
        for i in range(e):
            nc = -(-int(counts[i]) // 128)
            assert p[i] >= end, (counts, p)
            end = p[i] + 128 * nc
            assert end <= cap, (counts, p, cap)


def test_grouped_transpose_matches_exact_rederivation():
    rng = np.random.Generator(np.random.PCG64(5))
    counts = RAGGED
    off = _offsets(counts)
    x = (rng.standard_normal((int(off[-1]), 3)) * rng.choice([1e-3, 1.0, 40.0], size=(int(off[-1]), 1)))
    x = x.astype(np.float32)
    q_t, s_t, col_def, chunk_def = oracle.quant_transpose_grouped(x, off)
    p = oracle.padded_starts(off)
    for e in range(len(counts)):
        lo, hi = int(off[e]), int(off[e + 1])
        for g0 in range(lo, hi, 128):
            g1 = min(hi, g0 + 128)
            col = int(p[e] + (g0 - lo))
            for c in range(x.shape[1]):
                codes, s = exact_group(x[g0:g1, c])
                assert np.array_equal(q_t[c, col:col + (g1 - g0)], codes), (e, g0, c)
                assert s_t[c, col // 128] == s, (e, g0, c)
            if g1 - g0 < 128:                         # partial last group: zero padding
                assert np.all(q_t[:, col + (g1 - g0):col + 128] == 0)
                assert np.all(col_def[col:col + 128])
    assert chunk_def.sum() == sum(-(-c // 128) for c in counts)


def test_grouped_transpose_aligned_equals_plain():
    rng = np.random.Generator(np.random.PCG64(6))
    counts = [128, 0, 256, 384, 128]
    off = _offsets(counts)
    x = rng.standard_normal((int(off[-1]), 200)).astype(np.float32)
    q_t, s_t, _, _ = oracle.quant_transpose_grouped(x, off)
    qp, sp = oracle.quant_transpose(x)
    p = oracle.padded_starts(off)
    for e in range(len(counts)):
        lo, hi = int(off[e]), int(off[e + 1])
        assert np.array_equal(q_t[:, p[e]:p[e] + hi - lo], qp[:, lo:hi])
        assert np.array_equal(s_t[:, p[e] // 128:(p[e] + hi - lo) // 128], sp[:, lo // 128:hi // 128])


def _pow2_experts(counts, cols, rng):
    """Stack of per-expert blocks whose 128-token groups (counted from each
    expert's first token) are exactly quantizable; returns (float32, int*2^12)."""
    xs, ints = [], []
    for m in counts:
        if m == 0:
            continue
        a, ai = pow2_matrix(m, cols, (128, 1), rng)
        xs.append(a)
        ints.append(ai)
    return np.concatenate(xs), np.concatenate(ints)


def test_grouped_wgrad_closed_form():
    rng = np.random.Generator(np.random.PCG64(7))
    counts = [130, 0, 1, 255, 128]
    off = _offsets(counts)
    x, xi = _pow2_experts(counts, 256, rng)
    dy, dyi = _pow2_experts(counts, 128, rng)
    xq_t, xs_t, _, _ = oracle.quant_transpose_grouped(x, off)
    dyq_t, dys_t, _, _ = oracle.quant_transpose_grouped(dy, off)
    dw, s = oracle.grouped_wgrad_ref(dyq_t, dys_t, xq_t, xs_t, off)
    for e in range(len(counts)):
        lo, hi = int(off[e]), int(off[e + 1])
        if hi == lo:
            assert not dw[e].any()
            continue
        _close_to_exact(dw[e], s[e], dyi[lo:hi].T @ xi[lo:hi], 2.0 ** 24, hi - lo)


def test_grouped_wgrad_aligned_sums_to_dense():
    rng = np.random.Generator(np.random.PCG64(8))
    counts = [256, 128, 0, 384]
    off = _offsets(counts)
    x = rng.standard_normal((int(off[-1]), 256)).astype(np.float32)
    dy = (rng.standard_t(3, size=(int(off[-1]), 128))).astype(np.float32)
    gx = oracle.quant_transpose_grouped(x, off)
    gdy = oracle.quant_transpose_grouped(dy, off)
    dw, s = oracle.grouped_wgrad_ref(gdy[0], gdy[1], gx[0], gx[1], off)
    dense, sd = oracle.wgrad_ref(*oracle.quant_transpose(dy), *oracle.quant_transpose(x))
    assert np.allclose(dw.sum(0), dense, rtol=0, atol=1e-12 * sd.max())


def test_grouped_dgrad_closed_form():
    rng = np.random.Generator(np.random.PCG64(9))
    counts = [70, 0, 129, 1]
    off = _offsets(counts)
    n, k, e = 256, 384, len(counts)
    dy, dyi = pow2_matrix(int(off[-1]), n, (1, 128), rng)
    w, wi = pow2_matrix(e * n, k, (128, 128), rng)          # stacked [E*N, K]
    dyq, dys = oracle.quant_act_1x128(dy)
    wq, ws, wq_t = oracle.quant_weight_128x128(w)
    dx, s = oracle.grouped_dgrad_ref(dyq, dys, wq_t, ws, off)
    for i in range(e):
        lo, hi = int(off[i]), int(off[i + 1])
        if hi > lo:
            _close_to_exact(dx[lo:hi], s[lo:hi], dyi[lo:hi] @ wi[i * n:(i + 1) * n], 2.0 ** 24, n)


def test_grouped_dgrad_exact_rationals():
    x, w, offsets = synth.small_moe(300, 3, 256, 256, seed=21)
    off = offsets.numpy().astype(np.int64)
    e, n, k = w.shape
    rng = np.random.Generator(np.random.PCG64(22))
    dy = rng.standard_t(3, size=(int(off[-1]), n)).astype(np.float32)
    dyq, dys = oracle.quant_act_1x128(dy)
    wq, ws, wq_t = oracle.quant_weight_128x128(w.numpy().reshape(e * n, k))
    dx, s = oracle.grouped_dgrad_ref(dyq, dys, wq_t, ws, off)
    for _ in range(40):
        m = int(rng.integers(0, int(off[-1])))
        col = int(rng.integers(0, k))
        ex = int(np.searchsorted(off, m, side="right") - 1)
        # the output is the contraction over N of dY[m, :] and W_e[:, col]
        b = wq_t[col:col + 1, ex * n:(ex + 1) * n]
        sb = ws[ex * (n // 128):(ex + 1) * (n // 128), col // 128][None, :]
        want = oracle.exact_outputs(dyq[m:m + 1], dys[m:m + 1], b, sb, [(0, 0)])[0]
        assert abs(Fraction(float(dx[m, col])) - want) <= Fraction(n + 2) * Fraction(2) ** -53 * Fraction(
            float(s[m, col])) + Fraction(2) ** -1000


def test_grouped_wgrad_exact_rationals():
    rng = np.random.Generator(np.random.PCG64(23))
    counts = [200, 3, 0, 300]
    off = _offsets(counts)
    x = (rng.standard_normal((int(off[-1]), 256)) * 3).astype(np.float32)
    dy = rng.standard_t(3, size=(int(off[-1]), 128)).astype(np.float32)
    xq_t, xs_t, _, _ = oracle.quant_transpose_grouped(x, off)
    dyq_t, dys_t, _, _ = oracle.quant_transpose_grouped(dy, off)
    dw, s = oracle.grouped_wgrad_ref(dyq_t, dys_t, xq_t, xs_t, off)
    p = oracle.padded_starts(off)
    for _ in range(40):
        e = int(rng.choice([0, 1, 3]))
        nrow, kcol = int(rng.integers(0, 128)), int(rng.integers(0, 256))
        m = counts[e]
        nc = -(-m // 128)
        c0 = int(p[e]) // 128
        sl = slice(int(p[e]), int(p[e]) + 128 * nc)               # padding codes are 0
        want = oracle.exact_outputs(dyq_t[nrow:nrow + 1, sl], dys_t[nrow:nrow + 1, c0:c0 + nc],
                                    xq_t[kcol:kcol + 1, sl], xs_t[kcol:kcol + 1, c0:c0 + nc], [(0, 0)])[0]
        assert abs(Fraction(float(dw[e, nrow, kcol])) - want) <= Fraction(m + 2) * Fraction(2) ** -53 * Fraction(
            float(s[e, nrow, kcol])) + Fraction(2) ** -1000


def test_padding_codes_decode_to_zero():
    assert e4m3.decode(np.array([0], np.uint8))[0] == 0.0
