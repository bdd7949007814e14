"""The two workgroup tiles of the FP8 GEMM (256 x 128 with four waves, 256 x
256 with eight) run the same per-wave arithmetic in the same order, so their
outputs must agree bit for bit.  The library picks a tile by problem size;
fp8q_set_gemm_tile forces one.  Each case runs both tiles on the same operands
(the GPU quantizers' codes of seeded inputs) and compares the raw output bits;
one forced-wide case with a ragged tail is also checked against the oracle.
The 256 x 128 kernel is checked against the oracle in test_gpu_gemm.py."""

import numpy as np
import pytest
import torch

import fp8_fine_grained_quant_amd as fq
import oracle
import synth
from gpu_util import check_gemm, f32, gpu, log

pytestmark = pytest.mark.gpu


def _with_tile(tile, fn):
    fq.set_gemm_tile(tile)
    try:
        out = fn()
        torch.cuda.synchronize()
        return out
    finally:
        fq.set_gemm_tile("auto")


def _same_bits(fn, what):
    a = _with_tile("256x128", fn)
    b = _with_tile("256x256", fn)
    ia = a.view(torch.int16 if a.dtype == torch.bfloat16 else torch.int32)
    ib = b.view(torch.int16 if b.dtype == torch.bfloat16 else torch.int32)
    bad = int((ia != ib).sum())
    assert bad == 0, f"{what}: {bad} of {a.numel()} outputs differ between the two tiles"


def _operands(m, n, k, seed):
    x = synth.to_bf16(synth.general(m, k, seed=seed, kind="t3", outlier_frac=0.002, outlier_mul=40.0))
    w = torch.from_numpy((synth.general(n, k, seed=seed + 1) * 0.02).astype(np.float32))
    xq, xs = fq.quant_act_1x128(gpu(x))
    wq, ws, wq_t = fq.quant_weight_128x128(gpu(w))
    return x, w, xq, xs, wq, ws, wq_t


@pytest.mark.parametrize("m,n,k", [(1, 256, 128), (300, 256, 384), (257, 512, 1024), (513, 768, 256),
                                   (1000, 2048, 896), (4096, 2048, 7168)])
@pytest.mark.parametrize("out_dtype", [torch.bfloat16, torch.float32])
def test_fprop_tiles_agree(m, n, k, out_dtype):
    log(f"fprop {m}x{n}x{k} {out_dtype}")
    _, _, xq, xs, wq, ws, _ = _operands(m, n, k, seed=m + 3 * n + k)
    _same_bits(lambda: fq.gemm_fprop(xq, xs, wq, ws, out_dtype=out_dtype), f"fprop {m}x{n}x{k}")


@pytest.mark.parametrize("m,n,k", [(300, 384, 512), (1000, 1024, 2048), (4096, 2048, 7168)])
def test_dgrad_tiles_agree(m, n, k):
    """Dgrad reads the weight's block scales transposed (a different scale
    indexing from Fprop): dX [m, k] = dY [m, n] . W [n, k]."""
    log(f"dgrad {m}x{n}x{k}")
    dy = synth.to_bf16(synth.general(m, n, seed=m + n, kind="t3", outlier_frac=0.01, outlier_mul=100.0))
    w = torch.from_numpy((synth.general(n, k, seed=n + k) * 0.02).astype(np.float32))
    dyq, dys = fq.quant_act_1x128(gpu(dy))
    _, ws, wq_t = fq.quant_weight_128x128(gpu(w))
    _same_bits(lambda: fq.gemm_dgrad(dyq, dys, wq_t, ws), f"dgrad {m}x{n}x{k}")


@pytest.mark.parametrize("total,e,n,k", [(700, 5, 256, 512), (3000, 8, 512, 1024), (8192, 16, 1024, 2048)])
def test_grouped_tiles_agree(total, e, n, k):
    """Grouped Fprop and grouped Dgrad over ragged experts, including empty ones."""
    log(f"grouped {total} tokens, {e} experts, {n}x{k}")
    xm, wm, off = synth.small_moe(total, e, n, k, seed=total + e)
    xmq, xms = fq.quant_act_1x128(gpu(xm))
    wq, ws, wq_t = fq.quant_weight_128x128(gpu(wm).reshape(e * n, k))
    offg = gpu(off)
    _same_bits(lambda: fq.grouped_gemm(xmq, xms, wq.reshape(e, n, k), ws.reshape(e, n // 128, k // 128), offg),
               "grouped fprop")
    dym = synth.to_bf16(synth.general(total, n, seed=total + 1, kind="t3"))
    dyq, dys = fq.quant_act_1x128(gpu(dym))
    _same_bits(lambda: fq.grouped_gemm_dgrad(dyq, dys, wq_t, ws, offg), "grouped dgrad")


def test_wide_tile_against_oracle_ragged():
    m, n, k = 300, 512, 640
    x, w, xq, xs, wq, ws, _ = _operands(m, n, k, seed=91)
    y = _with_tile("256x256", lambda: fq.gemm_fprop(xq, xs, wq, ws, out_dtype=torch.float32))
    xo, xso = oracle.quant_act_1x128(f32(x))
    wo, wso, _ = oracle.quant_weight_128x128(f32(w))
    y_ref, s_ref = oracle.fprop_ref(xo, xso, wo, wso)
    check_gemm(f32(y), y_ref, s_ref, False, "wide fprop 300x512x640", False, nk=k // 128)


@pytest.mark.parametrize("t,n,k", [(128, 256, 256), (640, 512, 768), (4096, 2048, 7168)])
@pytest.mark.parametrize("accumulate", [False, True])
def test_wgrad_tiles_agree(t, n, k, accumulate):
    """dW [n, k] (=|+=) dY^T . X over t tokens: one B scale per output column."""
    log(f"wgrad T={t} {n}x{k} accumulate={accumulate}")
    x = synth.to_bf16(synth.general(t, k, seed=t + k, kind="t3", outlier_frac=0.002, outlier_mul=30.0))
    dy = synth.to_bf16(synth.general(t, n, seed=t + n + 1, kind="t3", outlier_frac=0.01, outlier_mul=100.0))
    xq_t, xs_t = fq.quant_transpose(gpu(x))
    dyq_t, dys_t = fq.quant_transpose(gpu(dy))
    base = torch.from_numpy(synth.general(n, k, seed=5).astype(np.float32))

    def run():
        dw = gpu(base.clone()) if accumulate else None
        return fq.gemm_wgrad(dyq_t, dys_t, xq_t, xs_t, dw)

    _same_bits(run, f"wgrad T={t} {n}x{k}")


@pytest.mark.parametrize("total,e,n,k", [(700, 5, 256, 512), (3000, 8, 512, 1024)])
def test_grouped_wgrad_tiles_agree(total, e, n, k):
    """Grouped Wgrad: ragged per-expert token chunks, an empty expert (its
    gradient written as zeros), per-expert outputs."""
    log(f"grouped wgrad {total} tokens, {e} experts, {n}x{k}")
    xm, _, off = synth.small_moe(total, e, n, k, seed=total + 2 * e)
    dym = synth.to_bf16(synth.general(total, n, seed=total + 3, kind="t3"))
    offg = gpu(off)
    xq_t, xs_t = fq.quant_transpose_grouped(gpu(xm), offg)
    dyq_t, dys_t = fq.quant_transpose_grouped(gpu(dym), offg)
    _same_bits(lambda: fq.grouped_gemm_wgrad(dyq_t, dys_t, xq_t, xs_t, offg, total), "grouped wgrad")


@pytest.mark.parametrize("m,n,k", [(300, 256, 512), (1000, 1024, 2048), (4096, 7168, 2048)])
@pytest.mark.parametrize("out", ["bf16", "f32_accumulate"])
def test_mx_tiles_agree(m, n, k, out):
    """The microscaling GEMM's two tiles: bit-identical outputs (BF16, and
    FP32 accumulated into an existing C).  K is a multiple of 512 so the
    scale rows are 16-byte aligned, which the 256 x 256 tile needs."""
    log(f"mx gemm {m}x{n}x{k} {out}")
    a = synth.to_bf16(synth.general(m, k, seed=m + k, kind="t3", outlier_frac=0.002, outlier_mul=30.0))
    b = torch.from_numpy((synth.general(n, k, seed=n + k + 1) * 0.02).astype(np.float32))
    aq, as_ = fq.quant_mx(gpu(a))
    bq, bs = fq.quant_mx(gpu(b))
    base = torch.from_numpy(synth.general(m, n, seed=9).astype(np.float32))

    def run():
        if out == "bf16":
            return fq.gemm_mx(aq, as_, bq, bs)
        return fq.gemm_mx(aq, as_, bq, bs, c=gpu(base.clone()))

    _same_bits(run, f"mx {m}x{n}x{k}")


def test_max_contraction_both_tiles():
    """The longest contraction a GEMM accepts (1024 chunks of 128): both
    tiles keep every chunk's block scales in LDS.  Bitwise agreement of the
    two tiles, and sampled rows against the oracle."""
    m, n, k = 300, 512, 1024 * 128
    log(f"fprop {m}x{n}x{k}")
    x, w, xq, xs, wq, ws, _ = _operands(m, n, k, seed=1234)
    _same_bits(lambda: fq.gemm_fprop(xq, xs, wq, ws, out_dtype=torch.float32), "fprop max K")
    rows = np.array([0, 1, 150, 255, 256, 299])
    y = _with_tile("256x256", lambda: fq.gemm_fprop(xq, xs, wq, ws, out_dtype=torch.float32))
    xo, xso = oracle.quant_act_1x128(f32(x[torch.from_numpy(rows)]))
    wo, wso, _ = oracle.quant_weight_128x128(f32(w))
    y_ref, s_ref = oracle.fprop_ref(xo, xso, wo, wso)
    check_gemm(f32(y)[rows], y_ref, s_ref, False, "wide fprop max K", False, nk=k // 128)
