"""GPU parity of the grouped (MoE) MX Fprop and Dgrad, fp8q_grouped_gemm_mx
and fp8q_grouped_gemm_mx_dgrad.

* Against the dense MX GEMM: every expert's rows of the grouped output equal,
  bit for bit, fp8q_gemm_mx on that expert's rows and weights (each output
  element takes the same instructions in the same order).  The dense MX GEMM
  is checked against the oracle in test_gpu_mx.py.
* Against the oracle: oracle.mx.gemm_mx_ref per expert on the same codes
  (the quantizers are bit-exact against oracle.mx), elementwise within the
  FP8 instruction's bound (gpu_util.check_gemm, exact=False, K/8 FP32
  additions).
* Dgrad: B is each expert's columns of the stacked weights' transposed codes
  (fp8q_quant_mx_transpose of [E*N, K]); the same two checks, with the dense
  MX GEMM on that strided column slice.
Cases: ragged experts with an empty one, an expert smaller than one tile,
one expert, K with unaligned (K % 512 != 0) and 16-byte aligned scale rows,
BF16 and FP32 output, and the MoE layer's full size (16384 tokens over 32
experts of [2048, 7168], Zipf counts with empty experts) on sampled rows."""

import numpy as np
import pytest
import torch

import fp8_fine_grained_quant_amd as fq
from oracle import mx
import synth
from gpu_util import check_gemm, f32, gpu, log, np_u8

pytestmark = pytest.mark.gpu


def _quantize(x, w):
    e, n, k = w.shape
    xq, xs = fq.quant_mx(gpu(x))
    wq, ws = fq.quant_mx(gpu(w).reshape(e * n, k))
    return xq, xs, wq.reshape(e, n, k), ws.reshape(e, n, k // 32)


def _same_as_dense(y, xq, xs, wq, ws, off, out_dtype, what):
    """Each expert's rows against the dense MX GEMM on them, bitwise."""
    iv = torch.int16 if out_dtype == torch.bfloat16 else torch.int32
    for e in range(wq.shape[0]):
        lo, hi = int(off[e]), int(off[e + 1])
        if hi == lo:
            continue
        yd = fq.gemm_mx(xq[lo:hi], xs[lo:hi], wq[e], ws[e], out_dtype=out_dtype)
        torch.cuda.synchronize()
        bad = int((y[lo:hi].view(iv) != yd.view(iv)).sum())
        assert bad == 0, f"{what}: expert {e} rows [{lo}, {hi}): {bad} outputs differ from the dense MX GEMM"


def _against_oracle(y, xq, xs, wq, ws, off, out_dtype, what, rows_per_expert=None):
    xq_n, xs_n, wq_n, ws_n = np_u8(xq), np_u8(xs), np_u8(wq), np_u8(ws)
    yf = f32(y)
    k = xq_n.shape[1]
    for e in range(wq_n.shape[0]):
        lo, hi = int(off[e]), int(off[e + 1])
        if hi == lo:
            continue
        rows = np.arange(lo, hi)
        if rows_per_expert is not None and len(rows) > rows_per_expert:
            # the expert's first and last rows, and rows across its tiles
            rows = np.unique(np.concatenate([rows[:2], rows[-2:],
                                             np.linspace(lo, hi - 1, rows_per_expert - 4).astype(np.int64)]))
        y_ref, s_ref = mx.gemm_mx_ref(xq_n[rows], xs_n[rows], wq_n[e], ws_n[e])
        check_gemm(yf[rows], y_ref, s_ref, out_dtype == torch.bfloat16, f"{what} expert {e}", exact=False,
                   nk=k // 8)


@pytest.mark.parametrize("total,e,n,k,dead", [(700, 5, 256, 512, 1), (3000, 8, 384, 1024, 2), (200, 1, 128, 384, 0),
                                              (1500, 6, 256, 640, 1), (90, 3, 128, 128, 1)])
@pytest.mark.parametrize("out_dtype", [torch.bfloat16, torch.float32])
def test_grouped_mx_ragged_experts(total, e, n, k, dead, out_dtype):
    log(f"grouped mx {total} tokens, {e} experts, {n}x{k}, {out_dtype}")
    x, w, off = synth.small_moe(total, e, n, k, seed=total + 7 * e + k, dead=dead)
    w = w * 50.0  # weights of O(1), so the E8M0 scales are not all the same
    xq, xs, wq, ws = _quantize(x, w)
    offg = gpu(off)
    y = fq.grouped_gemm_mx(xq, xs, wq, ws, offg, out_dtype=out_dtype)
    torch.cuda.synchronize()
    _same_as_dense(y, xq, xs, wq, ws, off, out_dtype, f"grouped mx {total}x{n}x{k}")
    _against_oracle(y, xq, xs, wq, ws, off, out_dtype, f"grouped mx {total}x{n}x{k}")


def test_grouped_mx_zero_tokens_and_deterministic():
    x, w, off = synth.small_moe(600, 4, 256, 512, seed=11)
    xq, xs, wq, ws = _quantize(x, w)
    offg = gpu(off)
    y1 = fq.grouped_gemm_mx(xq, xs, wq, ws, offg)
    y2 = fq.grouped_gemm_mx(xq, xs, wq, ws, offg)
    torch.cuda.synchronize()
    assert torch.equal(y1.view(torch.int16), y2.view(torch.int16))
    empty = torch.empty((0, 256), dtype=torch.bfloat16, device=y1.device)
    fq.fp8q_grouped_gemm_mx(xq[:0], xs[:0], wq, ws, gpu(torch.zeros(5, dtype=torch.int32)), empty)
    torch.cuda.synchronize()


def test_grouped_mx_moe_layer_full_size_sampled():
    """16384 tokens over 32 experts of [2048, 7168] (Zipf counts, 4 empty
    experts): every expert bitwise against the dense MX GEMM, and 12 rows per
    expert against the oracle."""
    log("grouped mx full size: 16384 tokens, 32 experts, 2048x7168")
    x, w, off = synth.moe_fprop()
    xq, xs, wq, ws = _quantize(x, w)
    del w
    offg = gpu(off)
    y = fq.grouped_gemm_mx(xq, xs, wq, ws, offg)
    torch.cuda.synchronize()
    _same_as_dense(y, xq, xs, wq, ws, off, torch.bfloat16, "grouped mx full size")
    _against_oracle(y, xq, xs, wq, ws, off, torch.bfloat16, "grouped mx full size", rows_per_expert=12)


# ---------------------------------------------------------------------- Dgrad
def _dgrad_operands(dy, w):
    e, n, k = w.shape
    dyq, dys = fq.quant_mx(gpu(dy))
    wq_t, ws_t = fq.quant_mx_transpose(gpu(w).reshape(e * n, k))
    return dyq, dys, wq_t, ws_t


def _dgrad_checks(dx, dyq, dys, wq_t, ws_t, off, out_dtype, what, rows_per_expert=None):
    iv = torch.int16 if out_dtype == torch.bfloat16 else torch.int32
    e_count = off.shape[0] - 1
    n = dyq.shape[1]
    dyq_n, dys_n, wq_n, ws_n = np_u8(dyq), np_u8(dys), np_u8(wq_t), np_u8(ws_t)
    dxf = f32(dx)
    for e in range(e_count):
        lo, hi = int(off[e]), int(off[e + 1])
        if hi == lo:
            continue
        bq, bs = wq_t[:, e * n:(e + 1) * n], ws_t[:, e * n // 32:(e + 1) * n // 32]  # strided views
        yd = fq.gemm_mx(dyq[lo:hi], dys[lo:hi], bq, bs, out_dtype=out_dtype)
        torch.cuda.synchronize()
        bad = int((dx[lo:hi].view(iv) != yd.view(iv)).sum())
        assert bad == 0, f"{what}: expert {e}: {bad} outputs differ from the dense MX GEMM"
        rows = np.arange(lo, hi)
        if rows_per_expert is not None and len(rows) > rows_per_expert:
            rows = np.unique(np.concatenate([rows[:2], rows[-2:],
                                             np.linspace(lo, hi - 1, rows_per_expert - 4).astype(np.int64)]))
        y_ref, s_ref = mx.gemm_mx_ref(dyq_n[rows], dys_n[rows], np.ascontiguousarray(wq_n[:, e * n:(e + 1) * n]),
                                      np.ascontiguousarray(ws_n[:, e * n // 32:(e + 1) * n // 32]))
        check_gemm(dxf[rows], y_ref, s_ref, out_dtype == torch.bfloat16, f"{what} expert {e}", exact=False,
                   nk=n // 8)


@pytest.mark.parametrize("total,e,n,k,dead", [(700, 5, 256, 384, 1), (3000, 8, 512, 1024, 2), (200, 1, 128, 256, 0),
                                              (90, 3, 384, 128, 1)])
@pytest.mark.parametrize("out_dtype", [torch.bfloat16, torch.float32])
def test_grouped_mx_dgrad_ragged_experts(total, e, n, k, dead, out_dtype):
    log(f"grouped mx dgrad {total} tokens, {e} experts, N={n} K={k}, {out_dtype}")
    _, w, off = synth.small_moe(total, e, n, k, seed=5 * total + e + n, dead=dead)
    dy = synth.to_bf16(synth.general(total, n, seed=total + n, kind="t3", outlier_frac=0.01, outlier_mul=100.0))
    dyq, dys, wq_t, ws_t = _dgrad_operands(dy, w * 50.0)
    dx = fq.grouped_gemm_mx_dgrad(dyq, dys, wq_t, ws_t, gpu(off), out_dtype=out_dtype)
    torch.cuda.synchronize()
    _dgrad_checks(dx, dyq, dys, wq_t, ws_t, off, out_dtype, f"grouped mx dgrad {total}x{n}x{k}")


def test_grouped_mx_dgrad_moe_backward_full_size_sampled():
    """dY [16384, 2048] over 32 experts of [2048, 7168] (Zipf counts, 4 empty
    experts) -> dX [16384, 7168]: every expert bitwise against the dense MX
    GEMM, 10 rows per expert against the oracle."""
    log("grouped mx dgrad full size: 16384 tokens, 32 experts, N=2048 K=7168")
    _, w, off = synth.moe_fprop()
    dy = synth.moe_dy()
    dyq, dys, wq_t, ws_t = _dgrad_operands(dy, w)
    del w
    dx = fq.grouped_gemm_mx_dgrad(dyq, dys, wq_t, ws_t, gpu(off))
    torch.cuda.synchronize()
    _dgrad_checks(dx, dyq, dys, wq_t, ws_t, off, torch.bfloat16, "grouped mx dgrad full size", rows_per_expert=10)
