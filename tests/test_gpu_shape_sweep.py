"""Seeded sweeps over shapes the fixed cases do not hit: every quantizer
(1x128, 128x128 with its transposed codes, transposing, dual, grouped
transposing) bit-exact against the oracle, and Fprop / Dgrad / Wgrad and their
grouped forms (FP8 and exact modes, BF16 and FP32 output, each workgroup tile)
against the oracle's float64 contraction at the bars of gpu_util.check_gemm.
Shapes are drawn from a counter-based generator per case, so every case is
reproducible from its id.  Sizes obey the interface's rules (16-byte row
strides for codes; GEMM contraction and output widths in multiples of 128)
and are otherwise ragged."""

import numpy as np
import pytest
import torch

import fp8_fine_grained_quant_amd as fq
import oracle
import synth
from gpu_util import assert_bytes_equal, assert_scales_equal, check_gemm, f32, gpu, log, np_u8

pytestmark = pytest.mark.gpu


def _rng(case):
    return np.random.Generator(np.random.PCG64(9000 + case))


def _tensor(rows, cols, seed, bf16, rng):
    kind = "t3" if rng.random() < 0.5 else "normal"
    x = synth.general(rows, cols, seed=seed, kind=kind, outlier_frac=0.003, outlier_mul=float(rng.choice([20, 80])))
    return synth.to_bf16(x) if bf16 else torch.from_numpy(x.astype(np.float32))


@pytest.mark.parametrize("case", range(48))
def test_quantizers_shape_sweep(case):
    rng = _rng(case)
    rows = int(rng.integers(1, 39)) * 16
    cols = int(rng.integers(1, 66)) * 16
    bf16 = bool(rng.random() < 0.5)
    log(f"quantizers case {case}: {rows}x{cols} {'bf16' if bf16 else 'fp32'}")
    x_cpu = _tensor(rows, cols, 100 + case, bf16, rng)
    x = gpu(x_cpu)
    xo = f32(x_cpu)

    q, s = fq.quant_act_1x128(x)
    qo, so = oracle.quant_act_1x128(xo)
    assert_bytes_equal(np_u8(q), qo, "act codes")
    assert_scales_equal(s.cpu().numpy(), so, "act scales")

    qw, sw, qwt = fq.quant_weight_128x128(x)
    wo, wso, wto = oracle.quant_weight_128x128(xo)
    assert_bytes_equal(np_u8(qw), wo, "weight codes")
    assert_bytes_equal(np_u8(qwt), wto, "weight transposed codes")
    assert_scales_equal(sw.cpu().numpy(), wso, "weight scales")

    qt, st = fq.quant_transpose(x)
    to, tso = oracle.quant_transpose(xo)
    assert_bytes_equal(np_u8(qt), to, "transpose codes")
    assert_scales_equal(st.cpu().numpy(), tso, "transpose scales")

    q2 = torch.empty_like(q)
    s2 = torch.empty_like(s)
    qt2 = torch.empty_like(qt)
    st2 = torch.empty_like(st)
    fq.fp8q_quant_act_transpose(x, q2, s2, qt2, st2)
    torch.cuda.synchronize()
    assert_bytes_equal(np_u8(q2), qo, "dual row codes")
    assert_scales_equal(s2.cpu().numpy(), so, "dual row scales")
    assert_bytes_equal(np_u8(qt2), to, "dual transposed codes")
    assert_scales_equal(st2.cpu().numpy(), tso, "dual transposed scales")


def _with_tile(tile, fn):
    fq.set_gemm_tile(tile)
    try:
        out = fn()
        torch.cuda.synchronize()
        return out
    finally:
        fq.set_gemm_tile("auto")


@pytest.mark.parametrize("case", range(48))
def test_gemms_shape_sweep(case):
    rng = _rng(100 + case)
    m = int(rng.integers(1, 700))
    n = int(rng.integers(1, 8)) * 128
    k = int(rng.integers(1, 15)) * 128
    exact = bool(rng.random() < 0.5)
    out_dtype = torch.float32 if rng.random() < 0.5 else torch.bfloat16
    tile = str(rng.choice(["auto", "256x128", "256x256"]))
    bf = out_dtype == torch.bfloat16
    log(f"gemm case {case}: m={m} n={n} k={k} exact={exact} out={out_dtype} tile={tile}")

    # Fprop Y [m, n] = X [m, k] . W [n, k]^T
    x = _tensor(m, k, 200 + case, True, rng)
    w = torch.from_numpy((synth.general(n, k, seed=300 + case) * 0.02).astype(np.float32))
    xq, xs = fq.quant_act_1x128(gpu(x))
    wq, ws, wq_t = fq.quant_weight_128x128(gpu(w))
    y = _with_tile(tile, lambda: fq.gemm_fprop(xq, xs, wq, ws, out_dtype=out_dtype, exact=exact))
    xo, xso = oracle.quant_act_1x128(f32(x))
    wo, wso, _ = oracle.quant_weight_128x128(f32(w))
    y_ref, s_ref = oracle.fprop_ref(xo, xso, wo, wso)
    check_gemm(f32(y), y_ref, s_ref, bf, f"sweep fprop {m}x{n}x{k}", exact, nk=k // 128)

    # Dgrad dX [m, k] = dY [m, n] . W [n, k]
    dy = _tensor(m, n, 400 + case, True, rng)
    dyq, dys = fq.quant_act_1x128(gpu(dy))
    dx = _with_tile(tile, lambda: fq.gemm_dgrad(dyq, dys, wq_t, ws, out_dtype=out_dtype, exact=exact))
    dyo, dyso = oracle.quant_act_1x128(f32(dy))
    y_ref, s_ref = oracle.dgrad_ref(dyo, dyso, wo, wso)
    check_gemm(f32(dx), y_ref, s_ref, bf, f"sweep dgrad {m}x{n}x{k}", exact, nk=n // 128)

    # Wgrad dW [nw, kw] = dY^T . X over t tokens (ragged output rows)
    t = int(rng.integers(1, 7)) * 128
    nw = int(rng.integers(1, 400))
    kw = int(rng.integers(1, 6)) * 128
    xw = _tensor(t, kw, 500 + case, True, rng)
    dyw = _tensor(t, nw, 600 + case, True, rng)
    buf = torch.zeros((t, nw + (-nw) % 8), dtype=torch.bfloat16)
    buf[:, :nw] = dyw
    xq_t, xs_t = fq.quant_transpose(gpu(xw))
    dq_t, ds_t = fq.quant_transpose(gpu(buf)[:, :nw])
    dw = _with_tile(tile, lambda: fq.gemm_wgrad(dq_t, ds_t, xq_t, xs_t, exact=exact))
    xto, xtso = oracle.quant_transpose(f32(xw))
    gto, gtso = oracle.quant_transpose(f32(dyw))
    y_ref, s_ref = oracle.wgrad_ref(gto, gtso, xto, xtso)
    check_gemm(f32(dw), y_ref, s_ref, False, f"sweep wgrad T={t} {nw}x{kw}", exact, nk=t // 128)


def _counts(rng, experts, tokens):
    """Ragged expert counts with about one expert in four empty."""
    cut = np.sort(rng.integers(0, tokens + 1, size=experts - 1))
    counts = np.diff(np.concatenate([[0], cut, [tokens]]))
    for e in range(experts):
        if rng.random() < 0.25 and experts > 1:  # a lone expert keeps every token
            nb = (e + 1) % experts
            counts[nb] += counts[e]
            counts[e] = 0
    assert counts.sum() == tokens
    return counts


@pytest.mark.parametrize("case", range(24))
def test_grouped_shape_sweep(case):
    """Grouped Fprop, grouped Dgrad (FP8 and exact where the entry point has
    it), the grouped transposing quantizer and grouped Wgrad over random
    expert counts, empty experts included."""
    rng = _rng(200 + case)
    experts = int(rng.integers(1, 10))
    tokens = int(rng.integers(1, 1500))
    counts = _counts(rng, experts, tokens)
    off = torch.tensor(np.concatenate([[0], np.cumsum(counts)]), dtype=torch.int32)
    n = int(rng.integers(1, 5)) * 128
    k = int(rng.integers(1, 6)) * 128
    exact = bool(rng.random() < 0.5)
    tile = str(rng.choice(["auto", "256x128", "256x256"]))
    log(f"grouped case {case}: counts {counts.tolist()} n={n} k={k} exact={exact} tile={tile}")
    og = gpu(off)
    offn = off.numpy()

    # grouped Fprop Y = X_e W_e^T
    x = _tensor(tokens, k, 700 + case, True, rng)
    w = torch.from_numpy((rng.standard_normal((experts * n, k)) * 0.02).astype(np.float32))
    xq, xs = fq.quant_act_1x128(gpu(x))
    wq, ws, wq_t = fq.quant_weight_128x128(gpu(w))
    y = _with_tile(tile, lambda: fq.grouped_gemm(xq, xs, wq.reshape(experts, n, k),
                                                 ws.reshape(experts, n // 128, k // 128), og, exact=exact))
    xo, xso = oracle.quant_act_1x128(f32(x))
    wo, wso, wo_t = oracle.quant_weight_128x128(f32(w))
    y_ref, s_ref = oracle.grouped_ref(xo, xso, wo.reshape(experts, n, k),
                                      wso.reshape(experts, n // 128, k // 128), offn)
    check_gemm(f32(y), y_ref, s_ref, True, f"sweep grouped fprop {counts.tolist()}", exact, nk=k // 128)

    # grouped Dgrad dX = dY_e W_e
    dy = _tensor(tokens, n, 800 + case, True, rng)
    dyq, dys = fq.quant_act_1x128(gpu(dy))
    dx = _with_tile(tile, lambda: fq.grouped_gemm_dgrad(dyq, dys, wq_t, ws, og))
    dyo, dyso = oracle.quant_act_1x128(f32(dy))
    y_ref, s_ref = oracle.grouped_dgrad_ref(dyo, dyso, wo_t, wso, offn)
    check_gemm(f32(dx), y_ref, s_ref, True, f"sweep grouped dgrad {counts.tolist()}", False, nk=n // 128)

    # grouped transposing quantizer and grouped Wgrad dW_e = dY_e^T X_e
    xq_t, xs_t = fq.quant_transpose_grouped(gpu(x), og)
    dq_t, ds_t = fq.quant_transpose_grouped(gpu(dy), og)
    gx = oracle.quant_transpose_grouped(f32(x), offn)
    gdy = oracle.quant_transpose_grouped(f32(dy), offn)
    col_def, chunk_def = gx[2], gx[3]
    assert_bytes_equal(np_u8(xq_t)[:, col_def], gx[0][:, col_def], "grouped transpose codes")
    assert_scales_equal(f32(xs_t)[:, chunk_def], gx[1][:, chunk_def], "grouped transpose scales")
    dw = _with_tile(tile, lambda: fq.grouped_gemm_wgrad(dq_t, ds_t, xq_t, xs_t, og, tokens))
    y_ref, s_ref = oracle.grouped_wgrad_ref(gdy[0], gdy[1], gx[0], gx[1], offn)
    nk = max(1, max(-(-int(c) // 128) for c in counts))
    check_gemm(f32(dw).reshape(-1, k), y_ref.reshape(-1, k), s_ref.reshape(-1, k), False,
               f"sweep grouped wgrad {counts.tolist()}", False, nk=nk)
