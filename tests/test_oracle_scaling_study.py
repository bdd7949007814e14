"""Numerics study of the scaling granularity (CPU, oracle arithmetic).

The pages motivate fine-grained scaling by outliers: per-tensor scaling maps
the tensor's max-abs to the FP8 maximum, so a few outliers push every other
value down into the coarse low range of E4M3 (the innerforce.co.kr excerpt,
paragraph on Figure 7 (a)); activation gradients have token-correlated
outliers, which 128x128 blocks (instead of 1x128 tiles) would spread over
128 tokens ("DeepSeek FP8 Training", last paragraph); delayed scaling takes
the scale from earlier iterations' max-abs ("unified E4M3 format" page,
"Dynamic Scaling and Online Quantization"), and a batch whose max exceeds
that history saturates.

On row samples of the linear-layer inputs (configs 2 and 3), each scheme is
applied with the same E4M3 rounding, and the error of the product against the
unquantized float64 product is measured.  The asserted orderings are what the
pages claim; the numbers are printed for the record.

The microscaling variant (MXFP8: 1x32 blocks along each product's
contraction axis, power-of-two E8M0 scales; the pages name such small-group
scaling as the hardware-supported counterpart, paragraph on Figure 7 (a)) is
measured the same way for Fprop, Dgrad and Wgrad.  The pages make no claim
about it, so only a property that follows from the definitions is asserted:
its power-of-two scale maps a block's max-abs into [256, 512), so a block
whose max-abs has a significand above 1.75 is clipped at 448 (its maximum
loses up to 1/8), which the method's scale (max-abs to exactly 448) never
does; and the block maximum's code is 448 exactly when that significand is
at least 1.6875 (432 lies halfway between the grid points 416 and 448 and
ties to the even code, 448)."""

import numpy as np
import pytest

import oracle
from oracle import e4m3, mx
from oracle.quant import group_scale
import synth

ROWS = 512


def _q_tensor(x, amax=None):
    """Per-tensor E4M3 quantization (one scale); returns the dequantized values."""
    x = np.asarray(x, np.float32)
    a = np.float32(np.abs(x).max()) if amax is None else np.float32(amax)
    s, inv = group_scale(a)
    return e4m3.decode(e4m3.encode(np.multiply(x, inv, dtype=np.float32))) * np.float64(s)


def _deq_rows(q, s):
    return e4m3.decode(q) * np.repeat(np.asarray(s, np.float64), 128, axis=1)[:, :q.shape[1]]


def _deq_blocks(q, s):
    s = np.repeat(np.repeat(np.asarray(s, np.float64), 128, axis=0), 128, axis=1)
    return e4m3.decode(q) * s[:q.shape[0], :q.shape[1]]


def _rel(y, ref):
    return float(np.linalg.norm(y - ref) / np.linalg.norm(ref))


@pytest.fixture(scope="module")
def linear():
    x, w = synth.linear_x_w()
    dy = synth.linear_dy()
    rng = np.random.Generator(np.random.PCG64(77))
    rows = np.sort(rng.choice(4096, size=ROWS, replace=False))
    other = np.setdiff1d(np.arange(4096), rows)[:ROWS]
    return (x.float().numpy()[rows], x.float().numpy()[other], w.numpy(),
            dy.float().numpy()[rows], dy.float().numpy()[other])


def test_fine_grained_beats_per_tensor_with_outlier_channels(linear):
    x, _, w, _, _ = linear
    ref = x.astype(np.float64) @ w.astype(np.float64).T
    xq, xs = oracle.quant_act_1x128(x)
    wq, ws, _ = oracle.quant_weight_128x128(w)
    fine = _rel(_deq_rows(xq, xs) @ _deq_blocks(wq, ws).T, ref)
    tensor = _rel(_q_tensor(x) @ _q_tensor(w).T, ref)
    print(f"\nFprop (config 2 rows, 2% channels x20): 1x128/128x128 {fine:.3e}, per-tensor {tensor:.3e}")
    # x20 outliers shift the per-tensor scale by ~4.3 bits only: the values
    # stay in E4M3's normal range, whose 3-bit mantissa dominates both errors
    assert fine < tensor


def test_fine_grained_beats_per_tensor_on_heavy_tailed_gradients(linear):
    """dY (Student-t(3), 1% of tokens x100) spans more than E4M3's 2^17.8
    dynamic range: per-tensor scaling flushes its small values to zero."""
    _, _, w, dy, _ = linear
    ref = dy.astype(np.float64) @ w.astype(np.float64)
    wq, ws, _ = oracle.quant_weight_128x128(w)
    wd = _deq_blocks(wq, ws)
    dq, ds = oracle.quant_act_1x128(dy)
    fine = _rel(_deq_rows(dq, ds) @ wd, ref)
    tensor = _rel(_q_tensor(dy) @ _q_tensor(w).T.T, ref)
    zero_t = float(np.mean(_q_tensor(dy) == 0))
    zero_f = float(np.mean(_deq_rows(dq, ds) == 0))
    print(f"\nDgrad (config 3 rows): 1x128 {fine:.3e} ({zero_f:.2%} zero codes), per-tensor {tensor:.3e} "
          f"({zero_t:.2%} zero codes)")
    assert fine < tensor and zero_f < zero_t


def test_token_tiles_beat_blocks_for_gradients_with_token_outliers(linear):
    _, _, w, dy, _ = linear
    ref = dy.astype(np.float64) @ w.astype(np.float64)
    wq, ws, _ = oracle.quant_weight_128x128(w)
    wd = _deq_blocks(wq, ws)
    dq, ds = oracle.quant_act_1x128(dy)
    tile = _rel(_deq_rows(dq, ds) @ wd, ref)
    bq, bs, _ = oracle.quant_weight_128x128(dy)        # the same rule over 128x128 blocks of dY
    block = _rel(_deq_blocks(bq, bs) @ wd, ref)
    print(f"\nDgrad (config 3 rows, 1% tokens x100): 1x128 {tile:.3e}, 128x128 {block:.3e}")
    assert tile < block


def test_delayed_scaling_saturates_when_the_batch_exceeds_its_history(linear):
    """Delayed scaling with a history whose max-abs is 4x below the current
    batch's (the batch's max grew since the history was taken): everything
    above the history's max saturates at 448, which online scaling avoids."""
    x, _, _, dy, _ = linear
    for name, cur in (("X", x), ("dY", dy)):
        ref = cur.astype(np.float64)
        hist = np.abs(cur).max() / 4
        online = _q_tensor(cur)
        delayed = _q_tensor(cur, amax=hist)
        sat = float(np.mean(np.abs(cur) > hist))
        e_on, e_del = _rel(online, ref), _rel(delayed, ref)
        e_fine = _rel(_deq_rows(*oracle.quant_act_1x128(cur)), ref)
        print(f"\n{name}: per-tensor online {e_on:.3e}, delayed (history max / 4) {e_del:.3e} with "
              f"{sat:.2e} of the values saturated, 1x128 online {e_fine:.3e}")
        assert e_fine < e_on < e_del


def _deq_mx(x):
    q, s = mx.quant_mx(np.asarray(x, np.float32))
    return mx.dequant_mx(q, s)


def _deq_mx_round_up(x):
    """1x32 blocks with the power-of-two scale rounded up instead,
    X = 2^ceil(log2(amax / 448)): the block maximum lands in (224, 448] and
    is never clipped (a study variant, not the OCP rule)."""
    x = np.asarray(x, np.float32)
    b = x.astype(np.float64).reshape(x.shape[0], -1, 32)
    amax = np.abs(b).max(axis=2, keepdims=True)
    X = np.exp2(np.ceil(np.log2(np.where(amax > 0, amax, 1.0) / 448.0)))
    return (e4m3.decode(e4m3.encode(b / X)) * X).reshape(x.shape)


def test_microscaling_error_beside_the_method(linear):
    x, _, w, dy, _ = linear
    x64, w64, dy64 = (a.astype(np.float64) for a in (x, w, dy))
    wq, ws, _ = oracle.quant_weight_128x128(w)
    wd = _deq_blocks(wq, ws)
    xq, xs = oracle.quant_act_1x128(x)
    dq, ds = oracle.quant_act_1x128(dy)
    rows = {}
    # Fprop Y = X W^T: both operands blocked along K
    ref = x64 @ w64.T
    rows["Fprop"] = (_rel(_deq_rows(xq, xs) @ wd.T, ref), _rel(_deq_mx(x) @ _deq_mx(w).T, ref),
                     _rel(_deq_mx_round_up(x) @ _deq_mx_round_up(w).T, ref))
    # Dgrad dX = dY W: blocked along N (W^T's rows for MX)
    ref = dy64 @ w64
    rows["Dgrad"] = (_rel(_deq_rows(dq, ds) @ wd, ref), _rel(_deq_mx(dy) @ _deq_mx(w.T).T, ref),
                     _rel(_deq_mx_round_up(dy) @ _deq_mx_round_up(w.T).T, ref))
    # Wgrad dW = dY^T X over the sampled tokens: blocked along the tokens
    ref = dy64.T @ x64
    dqt, dst = oracle.quant_transpose(dy)
    xqt, xst = oracle.quant_transpose(x)
    rows["Wgrad"] = (_rel(_deq_rows(dqt, dst) @ _deq_rows(xqt, xst).T, ref),
                     _rel(_deq_mx(dy.T) @ _deq_mx(x.T).T, ref),
                     _rel(_deq_mx_round_up(dy.T) @ _deq_mx_round_up(x.T).T, ref))
    for k, (meth, mxe, mxu) in rows.items():
        print(f"\n{k} (configs 2/3 rows): 1x128/128x128 {meth:.3e}, MXFP8 1x32 {mxe:.3e}, "
              f"1x32 with the scale rounded up {mxu:.3e}")
        assert 0 < meth < 0.1 and 0 < mxe < 0.1 and 0 < mxu < 0.1
    # the block maximum at the top of the grid: code 448 exactly when the
    # significand of the block's max-abs is >= 1.6875, clipped when > 1.75;
    # the method maps every group's max-abs to code 448 without clipping
    q, s = mx.quant_mx(x)
    amax = np.abs(x.astype(np.float64)).reshape(x.shape[0], -1, 32).max(axis=2)
    sig = amax / np.exp2(np.floor(np.log2(amax)))
    top = np.abs(e4m3.decode(q)).reshape(x.shape[0], -1, 32).max(axis=2)
    assert np.array_equal(top == 448.0, sig >= 1.6875)
    topv = top * mx.scale_value(s)
    clipped = sig > 1.75
    assert np.all(topv[clipped] < amax[clipped]) and np.all(topv[clipped] >= amax[clipped] * 0.875)
    assert np.abs(e4m3.decode(xq)).reshape(x.shape[0], -1, 128).max(axis=2).min() == 448.0
    print(f"MX blocks of X whose maximum is clipped at 448: {float(np.mean(clipped)):.3f}")
