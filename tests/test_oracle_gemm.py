"""Pins of the oracle's GEMM references.

* Closed form: operands built so that every group's max-abs is 448 * 2^e make
  quantization exact (s = 2^e, codes = the grid values), so each product must
  equal the plain integer matmul of the constructed matrices.  A wrong scale
  index, a transposed operand or a dropped term fails this.
* Exact rationals: the float64 references agree with the exact rational sum
  within the float64 summation bound.
"""

from fractions import Fraction

import numpy as np
import pytest

import oracle
from oracle import e4m3, quant
import synth

GRID = np.array([v for v in e4m3.decode(e4m3.finite_codes()) if abs(v) <= 448])


def pow2_matrix(rows, cols, grp, rng, emin=-3, emax=3):
    """Matrix whose (grp[0] x grp[1]) groups each hold grid values times 2^e
    (one random e per group) with at least one element of magnitude 448 * 2^e.
    Returns (float32 matrix, integer matrix equal to it times 2^12)."""
    m = rng.choice(GRID, size=(rows, cols))
    gr, gc = grp
    out = np.zeros((rows, cols))
    for r0 in range(0, rows, gr):
        for c0 in range(0, cols, gc):
            blk = m[r0:r0 + gr, c0:c0 + gc]
            i = rng.integers(blk.shape[0]), rng.integers(blk.shape[1])
            blk[i] = rng.choice([-448.0, 448.0])
            e = int(rng.integers(emin, emax + 1))
            out[r0:r0 + gr, c0:c0 + gc] = blk * 2.0 ** e
    ints = np.rint(out * 4096).astype(np.int64)
    assert np.array_equal(ints / 4096.0, out)
    return out.astype(np.float32), ints


def _close_to_exact(y, s, exact_ints, denom, k):
    want = exact_ints.astype(np.float64) / denom        # within 1/2 ulp of exact
    bound = (k + 2) * 2.0 ** -53 * s + 2.0 ** -1000
    err = np.abs(y - want)
    assert np.all(err <= bound), float((err / np.maximum(s, 1e-300)).max())


# ---------------------------------------------------------------- closed forms
def check_fprop_pow2(seed=0, m=130, n=256, k=384):
    rng = np.random.Generator(np.random.PCG64(seed))
    x, xi = pow2_matrix(m, k, (1, 128), rng)
    w, wi = pow2_matrix(n, k, (128, 128), rng)
    xq, xs = oracle.quant_act_1x128(x)
    wq, ws, _ = oracle.quant_weight_128x128(w)
    assert np.all(np.log2(xs) == np.rint(np.log2(xs)))      # exact powers of two
    y, s = oracle.fprop_ref(xq, xs, wq, ws)
    _close_to_exact(y, s, xi @ wi.T, 2.0 ** 24, k)


def check_dgrad_pow2(seed=1, m=70, n=256, k=384):
    rng = np.random.Generator(np.random.PCG64(seed))
    dy, dyi = pow2_matrix(m, n, (1, 128), rng)
    w, wi = pow2_matrix(n, k, (128, 128), rng)
    dyq, dys = oracle.quant_act_1x128(dy)
    wq, ws, _ = oracle.quant_weight_128x128(w)
    y, s = oracle.dgrad_ref(dyq, dys, wq, ws)
    _close_to_exact(y, s, dyi @ wi, 2.0 ** 24, n)


def check_wgrad_pow2(seed=2, t=256, n=128, k=384):
    rng = np.random.Generator(np.random.PCG64(seed))
    x, xi = pow2_matrix(t, k, (128, 1), rng)                 # groups of 128 tokens
    dy, dyi = pow2_matrix(t, n, (128, 1), rng)
    xq_t, xs_t = oracle.quant_transpose(x)
    dyq_t, dys_t = oracle.quant_transpose(dy)
    y, s = oracle.wgrad_ref(dyq_t, dys_t, xq_t, xs_t)
    _close_to_exact(y, s, dyi.T @ xi, 2.0 ** 24, t)


def check_grouped_pow2(seed=3, n=128, k=256):
    rng = np.random.Generator(np.random.PCG64(seed))
    offsets = np.array([0, 5, 5, 140, 141, 200], np.int64)   # expert 1 is empty
    e = len(offsets) - 1
    x, xi = pow2_matrix(int(offsets[-1]), k, (1, 128), rng)
    ws_all, wq_all, wis = [], [], []
    for _ in range(e):
        w, wi = pow2_matrix(n, k, (128, 128), rng)
        wq, ws, _ = oracle.quant_weight_128x128(w)
        wq_all.append(wq), ws_all.append(ws), wis.append(wi)
    xq, xs = oracle.quant_act_1x128(x)
    y, s = oracle.grouped_ref(xq, xs, np.stack(wq_all), np.stack(ws_all), offsets)
    want = np.zeros((int(offsets[-1]), n), np.int64)
    for i in range(e):
        lo, hi = offsets[i], offsets[i + 1]
        want[lo:hi] = xi[lo:hi] @ wis[i].T
    _close_to_exact(y, s, want, 2.0 ** 24, k)


def test_fprop_closed_form():
    check_fprop_pow2()


def test_dgrad_closed_form():
    check_dgrad_pow2()


def test_wgrad_closed_form():
    check_wgrad_pow2()


def test_grouped_closed_form():
    check_grouped_pow2()


# ------------------------------------------------------------- exact rationals
def _f64_close_to_fractions(y, s, pairs, exact, k):
    for (m, n), ex in zip(pairs, exact):
        err = abs(Fraction(float(y[m, n])) - ex)
        assert err <= Fraction((k + 2) * s[m, n]) * Fraction(2) ** -53 + Fraction(2) ** -1000, (m, n)


def check_tiny_config_exact():
    x, w = synth.tiny_fprop()
    xq, xs = oracle.quant_act_1x128(x.float().numpy())
    wq, ws, _ = oracle.quant_weight_128x128(w.numpy())
    y, s = oracle.fprop_ref(xq, xs, wq, ws)
    sb = ws[np.arange(128) // 128]                  # scale of (n, chunk)
    pairs = [(m, n) for m in range(128) for n in range(128)]
    exact = oracle.exact_outputs(xq, xs, wq, sb, pairs)
    _f64_close_to_fractions(y, s, pairs, exact, 256)


def test_tiny_config_all_outputs_exact():
    check_tiny_config_exact()


def test_dgrad_and_wgrad_exact_samples():
    rng = np.random.Generator(np.random.PCG64(4))
    dy = synth.to_bf16(synth.general(96, 256, seed=30, kind="t3")).float().numpy()
    w = (synth.general(256, 384, seed=31) * 0.02).astype(np.float32)
    dyq, dys = oracle.quant_act_1x128(dy)
    wq, ws, wq_t = oracle.quant_weight_128x128(w)
    y, s = oracle.dgrad_ref(dyq, dys, wq, ws)
    # the same product in NT form over the transposed weight codes
    sb = ws.T[np.arange(384) // 128]                # scale of (k_out, chunk over n)
    pairs = [(int(rng.integers(96)), int(rng.integers(384))) for _ in range(300)]
    _f64_close_to_fractions(y, s, pairs, oracle.exact_outputs(dyq, dys, wq_t, sb, pairs), 256)

    x = synth.to_bf16(synth.general(300, 200, seed=32)).float().numpy()
    g = synth.to_bf16(synth.general(300, 130, seed=33, kind="t3")).float().numpy()
    xq_t, xs_t = oracle.quant_transpose(x)
    gq_t, gs_t = oracle.quant_transpose(g)
    y, s = oracle.wgrad_ref(gq_t, gs_t, xq_t, xs_t)
    pairs = [(int(rng.integers(130)), int(rng.integers(200))) for _ in range(300)]
    _f64_close_to_fractions(y, s, pairs, oracle.exact_outputs(gq_t, gs_t, xq_t, xs_t, pairs), 300)


def test_brute_force_tiny_loops():
    """Pure-Python triple loop over decoded bytes on a 3x2x256 case."""
    x = synth.to_bf16(synth.general(3, 256, seed=40)).float().numpy()
    w = (synth.general(2, 256, seed=41) * 0.02).astype(np.float32)
    xq, xs = oracle.quant_act_1x128(x)
    wq, ws, _ = oracle.quant_weight_128x128(w)
    y, s = oracle.fprop_ref(xq, xs, wq, ws)
    for m in range(3):
        for n in range(2):
            tot = Fraction(0)
            for k in range(256):
                a = Fraction(float(e4m3.decode(xq[m, k:k + 1])[0])) * Fraction(float(xs[m, k // 128]))
                b = Fraction(float(e4m3.decode(wq[n, k:k + 1])[0])) * Fraction(float(ws[0, k // 128]))
                tot += a * b
            assert abs(Fraction(float(y[m, n])) - tot) <= Fraction(258 * float(s[m, n])) * Fraction(2) ** -53
