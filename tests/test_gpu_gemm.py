"""GPU parity of the block-scaled FP8 GEMMs against the oracle's float64
contraction of the dequantized operands, for both the FP8 matrix-instruction
entry points and the exact-accumulation (*_exact) ones.

Bars (elementwise, S = sum_k |a_k b_k|; see gpu_util.check_gemm): exact
variants FP32 |y - Y_ref| <= 1e-5 S, BF16 <= ulp_bf16(Y_ref) + 1e-5 S; FP8
variants within the bound implied by the FP8 instruction's 14-bit group
accumulation.  The operands of the GPU GEMM are the GPU quantizer's codes and
scales; the oracle quantizes the same seeded inputs itself (the quantizer
parity tests show the two agree bit for bit)."""

import numpy as np
import pytest
import torch

import fp8_fine_grained_quant_amd as fq
import oracle
import synth
from gpu_util import DEV, check_gemm, f32, gpu, log, sample_rows

pytestmark = pytest.mark.gpu

MODES = pytest.mark.parametrize("exact", [False, True], ids=["fp8", "exact"])


def _ref_rows_fprop(x_cpu, w_cpu, rows):
    xq, xs = oracle.quant_act_1x128(f32(x_cpu[torch.from_numpy(rows)]))
    wq, ws, _ = oracle.quant_weight_128x128(f32(w_cpu))
    return oracle.fprop_ref(xq, xs, wq, ws)


def _run_fprop(x_cpu, w_cpu, out_dtype, exact):
    x, w = gpu(x_cpu), gpu(w_cpu)
    xq, xs = fq.quant_act_1x128(x)
    wq, ws, _ = fq.quant_weight_128x128(w, transpose=False)
    y = fq.gemm_fprop(xq, xs, wq, ws, out_dtype=out_dtype, exact=exact)
    torch.cuda.synchronize()
    return y


# --------------------------------------------------------------------- Fprop
@MODES
@pytest.mark.parametrize("out_dtype", [torch.bfloat16, torch.float32])
def test_fprop_tiny_config_all_outputs(out_dtype, exact):
    x, w = synth.tiny_fprop()
    y = _run_fprop(x, w, out_dtype, exact)
    y_ref, s_ref = _ref_rows_fprop(x, w, np.arange(128))
    check_gemm(f32(y), y_ref, s_ref, out_dtype == torch.bfloat16, f"C1 fprop {out_dtype}", exact, nk=2)


@pytest.mark.parametrize("m,n,k", [(300, 384, 1024), (1, 128, 128), (257, 256, 384), (512, 128, 2048),
                                   (255, 640, 256)])
@pytest.mark.parametrize("out_dtype", [torch.bfloat16, torch.float32])
@MODES
def test_fprop_tiles_and_ragged_tail(m, n, k, out_dtype, exact):
    x = synth.to_bf16(synth.general(m, k, seed=m + n + k, outlier_frac=0.002, outlier_mul=30.0))
    w = torch.from_numpy((synth.general(n, k, seed=7 * k + n) * 0.02).astype(np.float32))
    y = _run_fprop(x, w, out_dtype, exact)
    y_ref, s_ref = _ref_rows_fprop(x, w, np.arange(m))
    check_gemm(f32(y), y_ref, s_ref, out_dtype == torch.bfloat16, f"fprop {m}x{n}x{k}", exact, nk=k // 128)


def test_fprop_output_guards_and_strided_output():
    m, n, k = 300, 256, 512
    x = synth.to_bf16(synth.general(m, k, seed=1))
    w = torch.from_numpy((synth.general(n, k, seed=2) * 0.02).astype(np.float32))
    xq, xs = fq.quant_act_1x128(gpu(x))
    wq, ws, _ = fq.quant_weight_128x128(gpu(w), transpose=False)
    ybuf = torch.full((m + 1, n + 64), 1234.0, dtype=torch.bfloat16, device=DEV)
    y = ybuf[:m, :n]
    fq.fp8q_gemm_fprop(xq, xs, wq, ws, y)
    torch.cuda.synchronize()
    assert torch.all(ybuf[:m, n:] == 1234.0) and torch.all(ybuf[m] == 1234.0)
    y_ref, s_ref = _ref_rows_fprop(x, w, np.arange(m))
    check_gemm(f32(y), y_ref, s_ref, True, "fprop strided", False, nk=4)


@MODES
def test_fprop_linear_config_full_size_sampled_rows(exact):
    x, w = synth.linear_x_w()
    log("C2 fprop 4096x2048x7168, 64 sampled rows")
    y = _run_fprop(x, w, torch.bfloat16, exact)
    rows = sample_rows(4096, 64, 11, must=(0, 255, 256, 4095))
    y_ref, s_ref = _ref_rows_fprop(x, w, rows)
    check_gemm(f32(y)[rows], y_ref, s_ref, True, "C2 fprop", exact, nk=56, strict=True)


@MODES
def test_fprop_deterministic(exact):
    x = gpu(synth.to_bf16(synth.general(512, 1024, seed=5)))
    w = gpu(torch.from_numpy((synth.general(256, 1024, seed=6) * 0.02).astype(np.float32)))
    xq, xs = fq.quant_act_1x128(x)
    wq, ws, _ = fq.quant_weight_128x128(w, transpose=False)
    y1 = fq.gemm_fprop(xq, xs, wq, ws, out_dtype=torch.float32, exact=exact)
    y2 = fq.gemm_fprop(xq, xs, wq, ws, out_dtype=torch.float32, exact=exact)
    assert torch.equal(y1, y2)


# --------------------------------------------------------------------- Dgrad
def _dgrad_case(dy_cpu, w_cpu, rows, exact, out_dtype=torch.bfloat16):
    dyq, dys = fq.quant_act_1x128(gpu(dy_cpu))
    wq, ws, wq_t = fq.quant_weight_128x128(gpu(w_cpu), transpose=True)
    dx = fq.gemm_dgrad(dyq, dys, wq_t, ws, out_dtype=out_dtype, exact=exact)
    torch.cuda.synchronize()
    dyo, dyso = oracle.quant_act_1x128(f32(dy_cpu[torch.from_numpy(rows)]))
    wo, wso, _ = oracle.quant_weight_128x128(f32(w_cpu))
    y_ref, s_ref = oracle.dgrad_ref(dyo, dyso, wo, wso)
    return f32(dx)[rows], y_ref, s_ref


@pytest.mark.parametrize("m,n,k", [(300, 512, 384), (1, 128, 128), (129, 256, 640)])
@pytest.mark.parametrize("out_dtype", [torch.bfloat16, torch.float32])
@MODES
def test_dgrad_tiles_and_ragged_tail(m, n, k, out_dtype, exact):
    dy = synth.to_bf16(synth.general(m, n, seed=m * 3 + n, kind="t3", outlier_frac=0.01, outlier_mul=100.0))
    w = torch.from_numpy((synth.general(n, k, seed=n + 5 * k) * 0.02).astype(np.float32))
    y, y_ref, s_ref = _dgrad_case(dy, w, np.arange(m), exact, out_dtype)
    check_gemm(y, y_ref, s_ref, out_dtype == torch.bfloat16, f"dgrad {m}x{n}x{k}", exact, nk=n // 128)


@MODES
def test_dgrad_linear_config_full_size_sampled_rows(exact):
    _, w = synth.linear_x_w()
    dy = synth.linear_dy()
    log("C3 dgrad 4096x7168 (contraction 2048), 64 sampled rows")
    rows = sample_rows(4096, 64, 12, must=(0, 4095))
    y, y_ref, s_ref = _dgrad_case(dy, w, rows, exact)
    check_gemm(y, y_ref, s_ref, True, "C3 dgrad", exact, nk=16, strict=True)


# --------------------------------------------------------------------- Wgrad
def _aligned_view(t):
    """The same matrix in a buffer whose row stride is a multiple of 16 bytes."""
    rows, cols = t.shape
    ld = cols + (-(cols * t.element_size()) % 16) // t.element_size()
    buf = torch.zeros((rows, ld), dtype=t.dtype, device=t.device)
    buf[:, :cols] = t
    return buf[:, :cols]


def _wgrad_case(x_cpu, dy_cpu, out_rows, exact, accumulate_into=None):
    xq_t, xs_t = fq.quant_transpose(_aligned_view(gpu(x_cpu)))
    dyq_t, dys_t = fq.quant_transpose(_aligned_view(gpu(dy_cpu)))
    dw = fq.gemm_wgrad(dyq_t, dys_t, xq_t, xs_t, dw=accumulate_into, exact=exact)
    torch.cuda.synchronize()
    xo, xso = oracle.quant_transpose(f32(x_cpu))
    go, gso = oracle.quant_transpose(f32(dy_cpu[:, torch.from_numpy(out_rows)]))
    y_ref, s_ref = oracle.wgrad_ref(go, gso, xo, xso)
    return dw, y_ref, s_ref


@pytest.mark.parametrize("t,n,k", [(512, 200, 384), (128, 1, 128), (256, 300, 256)])
@MODES
def test_wgrad_tiles_and_ragged_tail(t, n, k, exact):
    x = synth.to_bf16(synth.general(t, k, seed=t + k))
    dy = synth.to_bf16(synth.general(t, n, seed=t + n + 1, kind="t3", outlier_frac=0.01, outlier_mul=100.0))
    dw, y_ref, s_ref = _wgrad_case(x, dy, np.arange(n), exact)
    check_gemm(f32(dw), y_ref, s_ref, False, f"wgrad {t}x{n}x{k}", exact, nk=t // 128)


@MODES
def test_wgrad_accumulate(exact):
    t, n, k = 256, 130, 256
    x = synth.to_bf16(synth.general(t, k, seed=3))
    dy = synth.to_bf16(synth.general(t, n, seed=4))
    base = torch.from_numpy(synth.general(n, k, seed=5).astype(np.float32))
    dw, y_ref, s_ref = _wgrad_case(x, dy, np.arange(n), exact, accumulate_into=gpu(base.clone()))
    got = f32(dw).astype(np.float64) - base.numpy().astype(np.float64)
    # the stored sum adds one FP32 rounding of |base + y|, folded into S
    tol_extra = np.abs(base.numpy().astype(np.float64) + y_ref) * 2.0 ** -24
    check_gemm(got, y_ref, s_ref + tol_extra / 1e-5, False, "wgrad accumulate", exact, nk=2)


@MODES
def test_wgrad_linear_config_full_size_sampled_rows(exact):
    x, _ = synth.linear_x_w()
    dy = synth.linear_dy()
    log("C4 wgrad 2048x7168 over 4096 tokens, 48 sampled rows of dW")
    rows = sample_rows(2048, 48, 13, must=(0, 2047))
    dw, y_ref, s_ref = _wgrad_case(x, dy, rows, exact)
    check_gemm(f32(dw)[rows], y_ref, s_ref, False, "C4 wgrad", exact, nk=32)


# ------------------------------------------------------------------- Grouped
def _grouped_case(x_cpu, w_cpu, offsets, rows, exact, out_dtype=torch.bfloat16):
    e, n, k = w_cpu.shape
    xq, xs = fq.quant_act_1x128(gpu(x_cpu))
    wq, ws, _ = fq.quant_weight_128x128(gpu(w_cpu).reshape(e * n, k), transpose=False)
    y = fq.grouped_gemm(xq, xs, wq.reshape(e, n, k), ws.reshape(e, n // 128, k // 128), gpu(offsets),
                        out_dtype=out_dtype, exact=exact)
    torch.cuda.synchronize()
    off = offsets.numpy().astype(np.int64)
    y_ref = np.zeros((len(rows), n))
    s_ref = np.zeros((len(rows), n))
    xo, xso = oracle.quant_act_1x128(f32(x_cpu[torch.from_numpy(rows)]))
    experts = np.searchsorted(off, rows, side="right") - 1
    for ex in np.unique(experts):
        wo, wso, _ = oracle.quant_weight_128x128(f32(w_cpu[int(ex)]))
        sel = np.nonzero(experts == ex)[0]
        y_ref[sel], s_ref[sel] = oracle.fprop_ref(xo[sel], xso[sel], wo, wso)
    return f32(y)[rows], y_ref, s_ref, y, (xq, xs, wq, ws)


@pytest.mark.parametrize("tokens,experts,n,k,seed", [(700, 5, 256, 512, 1), (300, 8, 128, 256, 2),
                                                     (1000, 3, 384, 384, 3), (64, 4, 128, 128, 4)])
@MODES
def test_grouped_small_all_rows(tokens, experts, n, k, seed, exact):
    x, w, offsets = synth.small_moe(tokens, experts, n, k, seed)
    log(f"grouped tokens={tokens} experts={experts} counts={np.diff(offsets.numpy()).tolist()}")
    y, y_ref, s_ref, _, _ = _grouped_case(x, w, offsets, np.arange(tokens), exact)
    check_gemm(y, y_ref, s_ref, True, f"grouped {tokens}/{experts}", exact, nk=k // 128)


@MODES
def test_grouped_equals_per_expert_fprop(exact):
    x, w, offsets = synth.small_moe(900, 6, 256, 512, 9)
    _, _, _, y, (xq, xs, wq, ws) = _grouped_case(x, w, offsets, np.arange(1), exact)
    off = offsets.tolist()
    e, n, k = w.shape
    for i in range(e):
        lo, hi = off[i], off[i + 1]
        if hi == lo:
            continue
        ye = fq.gemm_fprop(xq[lo:hi], xs[lo:hi], wq[i * n:(i + 1) * n], ws[i * n // 128:(i + 1) * n // 128],
                           exact=exact)
        assert torch.equal(ye, y[lo:hi]), f"expert {i}"


@pytest.mark.timeout(600)
@MODES
def test_grouped_moe_config_sampled_rows(exact):
    x, w, offsets = synth.moe_fprop()
    off = offsets.numpy().astype(np.int64)
    counts = np.diff(off)
    log(f"C5 grouped 32 experts, counts {counts.tolist()}")
    live = np.nonzero(counts)[0]
    pick = sorted(set([int(live[np.argmin(counts[live])]), int(live[np.argmax(counts[live])]),
                       int(live[0]), int(live[-1])] + [int(v) for v in live[::9]]))
    rows = []
    for ex in pick:
        lo, hi = int(off[ex]), int(off[ex + 1])
        rows += [lo, hi - 1, (lo + hi) // 2] + list(range(lo + 250, min(hi, lo + 262)))
    rows = np.array(sorted(set(r for r in rows if 0 <= r < off[-1])), dtype=np.int64)
    log(f"checking experts {pick}, {len(rows)} rows")
    y, y_ref, s_ref, _, _ = _grouped_case(x, w, offsets, rows, exact)
    check_gemm(y, y_ref, s_ref, True, "C5 grouped", exact, nk=56, strict=True)
