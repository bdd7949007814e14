"""The quantizer fused into the epilogue of the GEMM that produces the next
layer's input: Fprop's Y and Dgrad's dX leave the GEMM in BF16 ("DeepSeek FP8
Training", Fprop list and input-gradient list) and are the next product's
1x128-quantized operand; activations are kept and passed on in FP8 (the
innerforce.co.kr excerpt of the DeepSeek-V3 report, FP8-framework paragraph).

Checks (GPU against GPU, so that no HIP output is ever an oracle input):
  * the fused call's BF16 output is bit-identical to the plain GEMM's, which
    test_gpu_gemm.py holds to the oracle;
  * its codes and scales are bit-identical to fp8q_quant_act_1x128 applied to
    that BF16 output, and that quantizer is bit-exact against the oracle
    (test_gpu_quant.py, test_gpu_quant_special.py);
  * the output rows it must not touch keep their guard values.
Both tiles (256x128 and 256x256) and both accumulation modes run."""

import numpy as np
import pytest
import torch

import fp8_fine_grained_quant_amd as fq
import synth
from gpu_util import DEV, gpu, log

pytestmark = pytest.mark.gpu

MODES = pytest.mark.parametrize("exact", [False, True], ids=["fp8", "exact"])


def _same(a, b, what):
    if a.dtype == torch.bfloat16:
        a, b = a.view(torch.int16), b.view(torch.int16)
    elif a.dtype == torch.float32:
        a, b = a.view(torch.int32), b.view(torch.int32)
    bad = int((a != b).sum())
    assert bad == 0, f"{what}: {bad} of {a.numel()} differ"


def _guarded(rows, cols, dtype, fill):
    """A [rows, cols] view into a guard-filled buffer with a wider row stride."""
    ld = cols + 32
    buf = torch.full((rows + 1, ld), fill, dtype=dtype, device=DEV)
    return buf, buf[:rows, :cols]


def _fprop_operands(m, n, k, seed, zero_rows=()):
    a = synth.general(m, k, seed=seed, kind="t3", outlier_frac=0.002, outlier_mul=40.0)
    a[list(zero_rows)] = 0.0
    x = synth.to_bf16(a)
    w = torch.from_numpy((synth.general(n, k, seed=seed + 1) * 0.02).astype(np.float32))
    xq, xs = fq.quant_act_1x128(gpu(x))
    wq, ws, wq_t = fq.quant_weight_128x128(gpu(w))
    return xq, xs, wq, ws, wq_t


def _check_fprop(m, n, k, exact, tile, seed, zero_rows=()):
    xq, xs, wq, ws, _ = _fprop_operands(m, n, k, seed, zero_rows)
    fq.set_gemm_tile(tile)
    try:
        y_plain = fq.gemm_fprop(xq, xs, wq, ws, exact=exact)
        ybuf, y = _guarded(m, n, torch.bfloat16, 7.0)
        qbuf, yq = _guarded(m, n, torch.uint8, 0xA5)
        sbuf, ys = _guarded(m, n // 128, torch.float32, -3.0)
        fq.fp8q_gemm_fprop_quant(xq, xs, wq, ws, y, yq, ys, exact=exact)
        _, yq2, ys2 = fq.gemm_fprop_quant(xq, xs, wq, ws, with_output=False, exact=exact)
    finally:
        fq.set_gemm_tile("auto")
    q_ref, s_ref = fq.quant_act_1x128(y_plain)
    torch.cuda.synchronize()
    _same(y, y_plain, "BF16 output")
    _same(yq, q_ref, "codes")
    _same(ys, s_ref, "scales")
    _same(yq2, q_ref, "codes (no BF16 output)")
    _same(ys2, s_ref, "scales (no BF16 output)")
    for buf, fill, what in ((ybuf, 7.0, "y"), (qbuf, 0xA5, "codes"), (sbuf, -3.0, "scales")):
        assert torch.all(buf[m] == fill) and torch.all(buf[:m, buf.shape[1] - 32:] == fill), what + " guards"
    return yq, ys


@MODES
@pytest.mark.parametrize("tile", ["256x128", "256x256"])
@pytest.mark.parametrize("m,n,k", [(1, 256, 128), (300, 256, 384), (513, 768, 1024), (1000, 2048, 896)])
def test_fprop_fused_quant(m, n, k, exact, tile):
    log(f"fprop_quant {m}x{n}x{k} {tile} exact={exact}")
    _check_fprop(m, n, k, exact, tile, seed=m + n + k)


@MODES
def test_fprop_fused_quant_linear_config(exact):
    """The linear layer's Fprop, X [4096,7168] . W [2048,7168]^T."""
    x, w = synth.linear_x_w()
    xq, xs = fq.quant_act_1x128(gpu(x))
    wq, ws, _ = fq.quant_weight_128x128(gpu(w), transpose=False)
    log(f"C2 fprop_quant exact={exact}")
    y_plain = fq.gemm_fprop(xq, xs, wq, ws, exact=exact)
    y, yq, ys = fq.gemm_fprop_quant(xq, xs, wq, ws, exact=exact)
    q_ref, s_ref = fq.quant_act_1x128(y_plain)
    torch.cuda.synchronize()
    _same(y, y_plain, "BF16 output")
    _same(yq, q_ref, "codes")
    _same(ys, s_ref, "scales")


def test_fprop_fused_quant_zero_rows():
    """Rows of X that are all zero give all-zero output rows: scale
    fl32(2^-100/448) and codes 0, as the quantizer gives them."""
    yq, ys = _check_fprop(300, 256, 384, False, "256x128", seed=5, zero_rows=(0, 17, 299))
    assert not yq[[0, 17, 299]].any()
    assert torch.all(ys[[0, 17, 299]] == torch.tensor(2.0 ** -100 / 448, dtype=torch.float32))


@MODES
@pytest.mark.parametrize("tile", ["256x128", "256x256"])
@pytest.mark.parametrize("m,n,k", [(300, 256, 512), (777, 384, 1024), (64, 128, 256)])
def test_dgrad_fused_quant(m, n, k, exact, tile):
    log(f"dgrad_quant {m}x{n}x{k} {tile} exact={exact}")
    dy = synth.to_bf16(synth.general(m, n, seed=m * 3 + n, kind="t3", outlier_frac=0.01, outlier_mul=100.0))
    w = torch.from_numpy((synth.general(n, k, seed=k) * 0.02).astype(np.float32))
    dyq, dys = fq.quant_act_1x128(gpu(dy))
    _, ws, wq_t = fq.quant_weight_128x128(gpu(w))
    fq.set_gemm_tile(tile)
    try:
        dx_plain = fq.gemm_dgrad(dyq, dys, wq_t, ws, exact=exact)
        dx, dxq, dxs = fq.gemm_dgrad_quant(dyq, dys, wq_t, ws, exact=exact)
    finally:
        fq.set_gemm_tile("auto")
    q_ref, s_ref = fq.quant_act_1x128(dx_plain)
    torch.cuda.synchronize()
    _same(dx, dx_plain, "BF16 output")
    _same(dxq, q_ref, "codes")
    _same(dxs, s_ref, "scales")


@MODES
def test_dgrad_fused_quant_linear_config(exact):
    """The linear layer's Dgrad, dY [4096,2048] . W [2048,7168]."""
    dy = synth.linear_dy()
    _, w = synth.linear_x_w()
    dyq, dys = fq.quant_act_1x128(gpu(dy))
    _, ws, wq_t = fq.quant_weight_128x128(gpu(w))
    log(f"C3 dgrad_quant exact={exact}")
    dx_plain = fq.gemm_dgrad(dyq, dys, wq_t, ws, exact=exact)
    dx, dxq, dxs = fq.gemm_dgrad_quant(dyq, dys, wq_t, ws, exact=exact)
    q_ref, s_ref = fq.quant_act_1x128(dx_plain)
    torch.cuda.synchronize()
    _same(dx, dx_plain, "BF16 output")
    _same(dxq, q_ref, "codes")
    _same(dxs, s_ref, "scales")
