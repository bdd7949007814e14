"""The binding refuses, before any call into the library, operands whose
shape or dtype does not match what the kernels will read or write through
raw pointers (CPU tensors: the check comes before the GPU-placement check,
so no device is needed)."""

import pytest
import torch

import fp8_fine_grained_quant_amd as fq

u8, f32, bf16, i32 = torch.uint8, torch.float32, torch.bfloat16, torch.int32


def z(*shape, dt=u8):
    return torch.zeros(*shape, dtype=dt)


def refused(fn, what):
    with pytest.raises((ValueError, TypeError)) as ei:
        fn()
    assert what in str(ei.value), str(ei.value)


def placed(fn):
    """Shapes accepted: the call gets as far as the GPU-placement check."""
    with pytest.raises(ValueError, match="GPU tensors only"):
        fn()


def test_quantizers():
    x = z(256, 384, dt=bf16)
    placed(lambda: fq.fp8q_quant_act_1x128(x, z(256, 384), z(256, 3, dt=f32)))
    refused(lambda: fq.fp8q_quant_act_1x128(x, z(256, 383), z(256, 3, dt=f32)), "q")
    refused(lambda: fq.fp8q_quant_act_1x128(x, z(256, 384), z(256, 2, dt=f32)), "scale")
    refused(lambda: fq.fp8q_quant_act_1x128(x, z(256, 384), z(256, 3, dt=bf16)), "scale")
    w = z(256, 384, dt=f32)
    placed(lambda: fq.fp8q_quant_weight_128x128(w, z(256, 384), z(384, 256), z(2, 3, dt=f32)))
    placed(lambda: fq.fp8q_quant_weight_128x128(w, z(256, 384), None, z(2, 3, dt=f32)))
    refused(lambda: fq.fp8q_quant_weight_128x128(w, z(256, 384), z(256, 384), z(2, 3, dt=f32)), "q_t")
    refused(lambda: fq.fp8q_quant_weight_128x128(w, z(256, 384), None, z(3, 2, dt=f32)), "scale")
    placed(lambda: fq.fp8q_quant_transpose(x, z(384, 256), z(384, 2, dt=f32)))
    refused(lambda: fq.fp8q_quant_transpose(x, z(256, 384), z(384, 2, dt=f32)), "q_t")
    refused(lambda: fq.fp8q_quant_transpose(x, z(384, 256), z(384, 3, dt=f32)), "scale_t")
    placed(lambda: fq.fp8q_quant_act_transpose(x, z(256, 384), z(256, 3, dt=f32), z(384, 256), z(384, 2, dt=f32)))
    refused(lambda: fq.fp8q_quant_act_transpose(x, z(256, 384), z(256, 3, dt=f32), z(384, 255),
                                                z(384, 2, dt=f32)), "q_t")
    off = z(5, dt=i32)
    cap = fq.token_capacity(256, 4)
    placed(lambda: fq.fp8q_quant_transpose_grouped(x, off, z(384, cap), z(384, cap // 128, dt=f32)))
    refused(lambda: fq.fp8q_quant_transpose_grouped(x, off, z(384, cap - 128), z(384, cap // 128, dt=f32)), "q_t")
    refused(lambda: fq.fp8q_quant_transpose_grouped(x, z(5, dt=torch.int64), z(384, cap),
                                                    z(384, cap // 128, dt=f32)), "offsets")


def test_gemms():
    m, n, k = 300, 256, 384
    xq, xs = z(m, k), z(m, 3, dt=f32)
    wq, ws, wq_t = z(n, k), z(2, 3, dt=f32), z(k, n)
    placed(lambda: fq.fp8q_gemm_fprop(xq, xs, wq, ws, z(m, n, dt=bf16)))
    refused(lambda: fq.fp8q_gemm_fprop(xq, xs, z(n, k - 128), ws, z(m, n, dt=bf16)), "wq")
    refused(lambda: fq.fp8q_gemm_fprop(xq, z(m, 2, dt=f32), wq, ws, z(m, n, dt=bf16)), "xs")
    refused(lambda: fq.fp8q_gemm_fprop(xq, xs, wq, z(3, 2, dt=f32), z(m, n, dt=bf16)), "ws")
    refused(lambda: fq.fp8q_gemm_fprop(xq, xs, wq, ws, z(m - 1, n, dt=bf16)), "y")
    dyq, dys = z(m, n), z(m, 2, dt=f32)
    placed(lambda: fq.fp8q_gemm_dgrad(dyq, dys, wq_t, ws, z(m, k, dt=bf16)))
    refused(lambda: fq.fp8q_gemm_dgrad(dyq, dys, wq, ws, z(m, k, dt=bf16)), "wq_t")
    refused(lambda: fq.fp8q_gemm_dgrad(dyq, dys, wq_t, ws, z(m, n, dt=bf16)), "dx")
    t = 384
    dyq_t, dys_t, xq_t, xs_t = z(n, t), z(n, 3, dt=f32), z(k, t), z(k, 3, dt=f32)
    placed(lambda: fq.fp8q_gemm_wgrad(dyq_t, dys_t, xq_t, xs_t, z(n, k, dt=f32)))
    refused(lambda: fq.fp8q_gemm_wgrad(dyq_t, dys_t, z(k, t - 128), xs_t, z(n, k, dt=f32)), "xq_t")
    refused(lambda: fq.fp8q_gemm_wgrad(dyq_t, dys_t, xq_t, xs_t, z(n, k, dt=bf16)), "dw")
    e = 4
    off = z(e + 1, dt=i32)
    wqe, wse = z(e, n, k), z(e, 2, 3, dt=f32)
    placed(lambda: fq.fp8q_grouped_gemm(xq, xs, wqe, wse, off, z(m, n, dt=bf16)))
    refused(lambda: fq.fp8q_grouped_gemm(xq, xs, wqe, z(e, 2, 2, dt=f32), off, z(m, n, dt=bf16)), "ws")
    refused(lambda: fq.fp8q_grouped_gemm(xq, xs, wqe, wse, z(e, dt=i32), z(m, n, dt=bf16)), "offsets")
    placed(lambda: fq.fp8q_grouped_gemm_dgrad(dyq, dys, z(k, e * n), z(e * 2, 3, dt=f32), off, z(m, k, dt=bf16)))
    refused(lambda: fq.fp8q_grouped_gemm_dgrad(dyq, dys, z(k, n), z(e * 2, 3, dt=f32), off, z(m, k, dt=bf16)),
            "wq_t")
    cap = fq.token_capacity(m, e)
    g_ops = (z(n, cap), z(n, cap // 128, dt=f32), z(k, cap), z(k, cap // 128, dt=f32))
    placed(lambda: fq.fp8q_grouped_gemm_wgrad(*g_ops, off, m, z(e, n, k, dt=f32)))
    refused(lambda: fq.fp8q_grouped_gemm_wgrad(*g_ops, off, m, z(e, n, k - 128, dt=f32)), "dw")
    refused(lambda: fq.fp8q_grouped_gemm_wgrad(g_ops[0], g_ops[1], z(k, cap + 128), g_ops[3], off, m,
                                               z(e, n, k, dt=f32)), "xq_t")


def test_microscaling():
    m, n, k = 300, 256, 384
    x = z(m, k, dt=bf16)
    placed(lambda: fq.fp8q_quant_mx_1x32(x, z(m, k), z(m, k // 32)))
    refused(lambda: fq.fp8q_quant_mx_1x32(x, z(m, k), z(m, k // 32 - 1)), "s")
    placed(lambda: fq.fp8q_quant_mx_transpose(x, z(k, m), z(k, 10)))
    refused(lambda: fq.fp8q_quant_mx_transpose(x, z(k, m), z(k, 10), z(m, k), None), "s")
    aq, as_, bq, bs = z(m, k), z(m, k // 32), z(n, k), z(n, k // 32 + 4)
    placed(lambda: fq.fp8q_gemm_mx(aq, as_, bq, bs, z(m, n, dt=bf16)))
    refused(lambda: fq.fp8q_gemm_mx(aq, z(m, k // 32 - 1), bq, bs, z(m, n, dt=bf16)), "as_")
    refused(lambda: fq.fp8q_gemm_mx(aq, as_, bq, bs, z(m, n + 128, dt=bf16)), "c")
    e, off = 4, z(5, dt=i32)
    placed(lambda: fq.fp8q_grouped_gemm_mx(aq, as_, z(e, n, k), z(e, n, k // 32), off, z(m, n, dt=bf16)))
    refused(lambda: fq.fp8q_grouped_gemm_mx(aq, as_, z(e, n, k), z(e, n, k // 16), off, z(m, n, dt=bf16)), "ws")
    dyq, dys = z(m, n), z(m, n // 32)
    placed(lambda: fq.fp8q_grouped_gemm_mx_dgrad(dyq, dys, z(k, e * n), z(k, e * n // 32), off, z(m, k, dt=bf16)))
    refused(lambda: fq.fp8q_grouped_gemm_mx_dgrad(dyq, dys, z(k, n), z(k, e * n // 32), off, z(m, k, dt=bf16)),
            "wq_t")
