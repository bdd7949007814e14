"""GPU parity of the three quantizers against the oracle: codes and scales
bit-exact, on the configurations' tensors and on edge shapes."""

import numpy as np
import pytest
import torch

import fp8_fine_grained_quant_amd as fq
import oracle
import synth
from gpu_util import DEV, assert_bytes_equal, assert_scales_equal, f32, gpu, log, np_u8, sample_rows

pytestmark = pytest.mark.gpu


def _padded(t, extra_cols=16, fill=0):
    """The same matrix inside a wider, guard-filled buffer (row stride > cols)."""
    rows, cols = t.shape
    esz = t.element_size()
    ld = cols + extra_cols
    ld += (-(ld * esz)) % 16 // esz
    buf = torch.full((rows + 1, ld), fill, dtype=t.dtype, device=t.device)
    buf[:rows, :cols] = t
    return buf, buf[:rows, :cols]


# ----------------------------------------------------------- activation 1x128
def _check_act(x_cpu, what, rows=None):
    x = gpu(x_cpu)
    q, s = fq.quant_act_1x128(x)
    torch.cuda.synchronize()
    xo = f32(x_cpu) if rows is None else f32(x_cpu[torch.from_numpy(rows)])
    qo, so = oracle.quant_act_1x128(xo)
    qg, sg = np_u8(q), s.cpu().numpy()
    if rows is not None:
        qg, sg = qg[rows], sg[rows]
    assert_bytes_equal(qg, qo, what + " codes")
    assert_scales_equal(sg, so, what + " scales")
    return q, s


def test_act_tiny_config():
    x, _ = synth.tiny_fprop()
    _check_act(x, "C1 X")


def test_act_linear_x_full_size_sampled_rows():
    x, _ = synth.linear_x_w()
    log("C2 X [4096,7168] quant_act, 256 sampled rows")
    _check_act(x, "C2 X", rows=sample_rows(4096, 256, 1, must=(0, 4095)))


def test_act_linear_dy_full():
    dy = synth.linear_dy()
    log("C3 dY [4096,2048] quant_act, all rows")
    _check_act(dy, "C3 dY")


def test_act_moe_x_full_size_sampled_rows():
    rng = np.random.Generator(np.random.PCG64(55))
    x = synth.to_bf16(rng.standard_normal((16384, 7168), dtype=np.float32))
    log("[16384,7168] quant_act, 256 sampled rows")
    _check_act(x, "MoE-size X", rows=sample_rows(16384, 256, 2, must=(0, 16383)))


@pytest.mark.parametrize("shape", [(1, 1), (1, 128), (3, 130), (5, 7), (257, 1000), (64, 4096 + 8)])
@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
def test_act_edge_shapes_with_guards(shape, dtype):
    rows, cols = shape
    a = synth.general(rows, cols, seed=rows * 1000 + cols, kind="t3", outlier_frac=0.01, outlier_mul=300.0)
    x_cpu = torch.from_numpy(a.astype(np.float32)).to(dtype)
    xbuf, x = _padded(gpu(x_cpu))
    qbuf = torch.full((rows + 1, ((cols + 15) // 16) * 16 + 16), 0xA5, dtype=torch.uint8, device=DEV)
    sbuf = torch.full((rows + 1, (cols + 127) // 128 + 1), -7.0, dtype=torch.float32, device=DEV)
    q, s = qbuf[:rows, :cols], sbuf[:rows, :(cols + 127) // 128]
    fq.fp8q_quant_act_1x128(x, q, s)
    torch.cuda.synchronize()
    qo, so = oracle.quant_act_1x128(f32(x_cpu))
    assert_bytes_equal(np_u8(q), qo, f"{shape} codes")
    assert_scales_equal(s.cpu().numpy(), so, f"{shape} scales")
    # guards: nothing written outside the views
    assert torch.all(qbuf[:rows, cols:] == 0xA5) and torch.all(qbuf[rows] == 0xA5)
    assert torch.all(sbuf[:rows, (cols + 127) // 128:] == -7.0) and torch.all(sbuf[rows] == -7.0)


@pytest.mark.parametrize("shape", [(1, 128), (3, 384), (257, 1024), (129, 2048), (7, 7168)])
@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
def test_act_dense_shapes_with_guards(shape, dtype):
    """Dense tensors (row stride = cols, a multiple of 128) take the flat
    indexing path; group counts that do not fill the last wave check its tail."""
    rows, cols = shape
    a = synth.general(rows, cols, seed=rows * 7 + cols, kind="t3", outlier_frac=0.01, outlier_mul=300.0)
    x_cpu = torch.from_numpy(a.astype(np.float32)).to(dtype)
    xbuf = torch.full((rows + 1, cols), 5.0, dtype=dtype, device=DEV)
    xbuf[:rows] = gpu(x_cpu)
    x = xbuf[:rows]
    g = cols // 128
    qbuf = torch.full((rows + 1, cols), 0xA5, dtype=torch.uint8, device=DEV)
    sbuf = torch.full((rows + 1, g), -7.0, dtype=torch.float32, device=DEV)
    q, s = qbuf[:rows], sbuf[:rows]
    fq.fp8q_quant_act_1x128(x, q, s)
    torch.cuda.synchronize()
    qo, so = oracle.quant_act_1x128(f32(x_cpu))
    assert_bytes_equal(np_u8(q), qo, f"{shape} codes")
    assert_scales_equal(s.cpu().numpy(), so, f"{shape} scales")
    assert torch.all(qbuf[rows] == 0xA5) and torch.all(sbuf[rows] == -7.0)


def test_act_special_groups():
    x = np.zeros((8, 512), np.float32)
    x[1, :] = -0.0                                       # signed zeros
    x[2, :] = 3.0                                        # constant group
    x[3, :128] = np.float32(3e38)                        # extreme max-abs (fp32 input)
    x[3, 128:256] = np.float32(1e-38)                    # tiny max-abs
    x[3, 256:384] = np.float32(1e-44)                    # below the 2^-100 floor, denormal
    x[4, ::2] = -1e-3
    x[4, 1::2] = 1e-45                                   # mixed signs, denormal
    rng = np.random.Generator(np.random.PCG64(9))
    x[5] = rng.standard_normal(512).astype(np.float32) * np.float32(2.0 ** 60)
    x[6] = rng.standard_normal(512).astype(np.float32) * np.float32(2.0 ** -60)
    x[7, 5] = 448.0 * 2.0 ** -3
    xt = torch.from_numpy(x)
    _check_act(xt, "special fp32")
    xb = torch.from_numpy(np.clip(x, -3e38, 3e38)).to(torch.bfloat16)
    _check_act(xb, "special bf16")


def test_act_deterministic():
    dy = gpu(synth.linear_dy(m=512, n=2048))
    q1, s1 = fq.quant_act_1x128(dy)
    q2, s2 = fq.quant_act_1x128(dy)
    assert torch.equal(q1, q2) and torch.equal(s1, s2)


# ------------------------------------------------------------- weight 128x128
def _check_weight(w_cpu, what):
    w = gpu(w_cpu)
    q, s, q_t = fq.quant_weight_128x128(w)
    torch.cuda.synchronize()
    qo, so, qto = oracle.quant_weight_128x128(f32(w_cpu))
    assert_bytes_equal(np_u8(q), qo, what + " codes")
    assert_scales_equal(s.cpu().numpy(), so, what + " scales")
    assert_bytes_equal(np_u8(q_t), qto, what + " transposed codes")
    assert torch.equal(q_t, q.t())


def test_weight_tiny_config():
    _, w = synth.tiny_fprop()
    _check_weight(w, "C1 W")


def test_weight_linear_full():
    _, w = synth.linear_x_w()
    log("C2 W [2048,7168] quant_weight with q_t, all blocks")
    _check_weight(w, "C2 W")


@pytest.mark.parametrize("shape", [(1, 1), (130, 140), (1, 300), (300, 1), (257, 384), (128, 4)])
@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
def test_weight_edge_shapes(shape, dtype):
    a = synth.general(*shape, seed=shape[0] * 7 + shape[1]) * 0.02
    w_cpu = torch.from_numpy(a.astype(np.float32)).to(dtype)
    rows, cols = shape
    wbuf, w = _padded(gpu(w_cpu))
    ldq = ((cols + 15) // 16) * 16 + 16
    ldqt = ((rows + 15) // 16) * 16 + 16
    qbuf = torch.full((rows + 1, ldq), 0x5A, dtype=torch.uint8, device=DEV)
    qtbuf = torch.full((cols + 1, ldqt), 0x5A, dtype=torch.uint8, device=DEV)
    gs = ((rows + 127) // 128, (cols + 127) // 128)
    sbuf = torch.full((gs[0] + 1, gs[1] + 1), -3.0, dtype=torch.float32, device=DEV)
    q, q_t, s = qbuf[:rows, :cols], qtbuf[:cols, :rows], sbuf[:gs[0], :gs[1]]
    fq.fp8q_quant_weight_128x128(w, q, q_t, s)
    torch.cuda.synchronize()
    qo, so, qto = oracle.quant_weight_128x128(f32(w_cpu))
    assert_bytes_equal(np_u8(q), qo, f"{shape} codes")
    assert_bytes_equal(np_u8(q_t), qto, f"{shape} q_t")
    assert_scales_equal(s.cpu().numpy(), so, f"{shape} scales")
    assert torch.all(qbuf[:rows, cols:] == 0x5A) and torch.all(qbuf[rows] == 0x5A)
    assert torch.all(qtbuf[:cols, rows:] == 0x5A) and torch.all(qtbuf[cols] == 0x5A)
    assert torch.all(sbuf[gs[0]] == -3.0) and torch.all(sbuf[:, gs[1]] == -3.0)


def test_weight_without_transpose_and_stacked_experts():
    """The MoE weights are quantized as one stacked [E*N, K] matrix; blocks
    never straddle experts because N % 128 == 0.  Checked on 3 experts of
    [2048, 7168] against per-expert oracle quantization."""
    rng = np.random.Generator(np.random.PCG64(77))
    e, n, k = 3, 2048, 7168
    w_cpu = torch.from_numpy((rng.standard_normal((e, n, k), dtype=np.float32) * np.float32(0.02)))
    w = gpu(w_cpu).reshape(e * n, k)
    q, s, q_t = fq.quant_weight_128x128(w, transpose=False)
    torch.cuda.synchronize()
    assert q_t is None
    qg, sg = np_u8(q).reshape(e, n, k), s.cpu().numpy().reshape(e, n // 128, k // 128)
    for i in range(e):
        qo, so, _ = oracle.quant_weight_128x128(w_cpu[i].numpy())
        assert_bytes_equal(qg[i], qo, f"expert {i} codes")
        assert_scales_equal(sg[i], so, f"expert {i} scales")


def test_weight_stacked_experts_above_64mb_with_transpose():
    """Code arrays above 64 MB are written non-temporally: 5 stacked experts
    of [2048, 7168] (73 M codes), with the transposed codes, against the
    oracle on the first and last expert."""
    rng = np.random.Generator(np.random.PCG64(78))
    e, n, k = 5, 2048, 7168
    w_cpu = torch.from_numpy((rng.standard_normal((e, n, k), dtype=np.float32) * np.float32(0.02)))
    w = gpu(w_cpu).reshape(e * n, k)
    q, s, q_t = fq.quant_weight_128x128(w)
    torch.cuda.synchronize()
    qg, sg = np_u8(q).reshape(e, n, k), s.cpu().numpy().reshape(e, n // 128, k // 128)
    for i in (0, e - 1):
        log(f"stacked expert {i} of {e}")
        qo, so, qto = oracle.quant_weight_128x128(w_cpu[i].numpy())
        assert_bytes_equal(qg[i], qo, f"expert {i} codes")
        assert_scales_equal(sg[i], so, f"expert {i} scales")
        assert_bytes_equal(np_u8(q_t[:, i * n:(i + 1) * n]), qto, f"expert {i} transposed codes")


# ------------------------------------------------------------- quant transpose
def _check_transpose(x_cpu, what, cols=None):
    x = gpu(x_cpu)
    q_t, s_t = fq.quant_transpose(x)
    torch.cuda.synchronize()
    xo = f32(x_cpu) if cols is None else f32(x_cpu[:, torch.from_numpy(cols)])
    qo, so = oracle.quant_transpose(xo)
    qg, sg = np_u8(q_t), s_t.cpu().numpy()
    if cols is not None:
        qg, sg = qg[cols], sg[cols]
    assert_bytes_equal(qg, qo, what + " codes")
    assert_scales_equal(sg, so, what + " scales")
    return q_t, s_t


def test_transpose_wgrad_x_full_size_sampled_channels():
    x, _ = synth.linear_x_w()
    log("C4 X [4096,7168] quant_transpose, 384 sampled channels")
    _check_transpose(x, "C4 X^T", cols=sample_rows(7168, 384, 3, must=(0, 7167)))


def test_transpose_wgrad_dy_full():
    dy = synth.linear_dy()
    log("C4 dY [4096,2048] quant_transpose, all channels")
    _check_transpose(dy, "C4 dY^T")


@pytest.mark.parametrize("shape", [(1, 1), (128, 128), (300, 70), (1, 5), (257, 129), (129, 1), (1000, 24)])
@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
def test_transpose_edge_shapes_with_guards(shape, dtype):
    rows, cols = shape
    a = synth.general(rows, cols, seed=rows + 31 * cols, kind="t3", outlier_frac=0.02, outlier_mul=100.0)
    x_cpu = torch.from_numpy(a.astype(np.float32)).to(dtype)
    xbuf, x = _padded(gpu(x_cpu))
    ldqt = ((rows + 15) // 16) * 16 + 16
    qtbuf = torch.full((cols + 1, ldqt), 0x3C, dtype=torch.uint8, device=DEV)
    g = (rows + 127) // 128
    sbuf = torch.full((cols + 1, g + 1), -5.0, dtype=torch.float32, device=DEV)
    q_t, s_t = qtbuf[:cols, :rows], sbuf[:cols, :g]
    fq.fp8q_quant_transpose(x, q_t, s_t)
    torch.cuda.synchronize()
    qo, so = oracle.quant_transpose(f32(x_cpu))
    assert_bytes_equal(np_u8(q_t), qo, f"{shape} codes")
    assert_scales_equal(s_t.cpu().numpy(), so, f"{shape} scales")
    assert torch.all(qtbuf[:cols, rows:] == 0x3C) and torch.all(qtbuf[cols] == 0x3C)
    assert torch.all(sbuf[cols] == -5.0) and torch.all(sbuf[:, g] == -5.0)


def test_transpose_equals_act_of_transposed_on_gpu():
    dy = gpu(synth.linear_dy(m=640, n=384))
    q_t, s_t = fq.quant_transpose(dy)
    q2, s2 = fq.quant_act_1x128(dy.t().contiguous())
    assert torch.equal(q_t, q2) and torch.equal(s_t, s2)


# ------------------------------------------------------- dual-output quantizer
@pytest.mark.parametrize("shape", [(1, 1), (128, 128), (300, 70), (1, 5), (257, 129), (129, 1), (1000, 24),
                                   (130, 300)])
@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
def test_act_transpose_edge_shapes_with_guards(shape, dtype):
    rows, cols = shape
    a = synth.general(rows, cols, seed=rows + 17 * cols, kind="t3", outlier_frac=0.02, outlier_mul=100.0)
    x_cpu = torch.from_numpy(a.astype(np.float32)).to(dtype)
    _, x = _padded(gpu(x_cpu))
    r16 = lambda n: ((n + 15) // 16) * 16 + 16
    g_r, g_c = (cols + 127) // 128, (rows + 127) // 128
    qbuf = torch.full((rows + 1, r16(cols)), 0x3C, dtype=torch.uint8, device=DEV)
    sbuf = torch.full((rows + 1, g_r + 1), -5.0, dtype=torch.float32, device=DEV)
    qtbuf = torch.full((cols + 1, r16(rows)), 0x3C, dtype=torch.uint8, device=DEV)
    stbuf = torch.full((cols + 1, g_c + 1), -5.0, dtype=torch.float32, device=DEV)
    q, s, q_t, s_t = qbuf[:rows, :cols], sbuf[:rows, :g_r], qtbuf[:cols, :rows], stbuf[:cols, :g_c]
    fq.fp8q_quant_act_transpose(x, q, s, q_t, s_t)
    torch.cuda.synchronize()
    qo, so = oracle.quant_act_1x128(f32(x_cpu))
    qto, sto = oracle.quant_transpose(f32(x_cpu))
    assert_bytes_equal(np_u8(q), qo, f"{shape} row codes")
    assert_scales_equal(s.cpu().numpy(), so, f"{shape} row scales")
    assert_bytes_equal(np_u8(q_t), qto, f"{shape} transposed codes")
    assert_scales_equal(s_t.cpu().numpy(), sto, f"{shape} transposed scales")
    for buf, r, c, fill in ((qbuf, rows, cols, 0x3C), (qtbuf, cols, rows, 0x3C), (sbuf, rows, g_r, -5.0),
                            (stbuf, cols, g_c, -5.0)):
        assert torch.all(buf[:r, c:] == fill) and torch.all(buf[r] == fill)


@pytest.mark.parametrize("which", ["C2 X", "C3 dY"])
def test_act_transpose_equals_the_two_quantizers_full_size(which):
    x = gpu(synth.linear_x_w()[0] if which == "C2 X" else synth.linear_dy())
    log(f"{which} dual-output quantizer against quant_act_1x128 + quant_transpose")
    q, s, q_t, s_t = fq.quant_act_transpose(x)
    q1, s1 = fq.quant_act_1x128(x)
    q2, s2 = fq.quant_transpose(x)
    torch.cuda.synchronize()
    assert torch.equal(q, q1) and torch.equal(s, s1)
    assert torch.equal(q_t, q2) and torch.equal(s_t, s2)
    rows = sample_rows(x.shape[0], 32, 5, must=(0, x.shape[0] - 1))
    qo, so = oracle.quant_act_1x128(f32(x[torch.from_numpy(rows).to(DEV)]))
    assert_bytes_equal(np_u8(q)[rows], qo, which + " row codes (sampled rows)")
    assert_scales_equal(s.cpu().numpy()[rows], so, which + " row scales (sampled rows)")
