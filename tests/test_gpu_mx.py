"""GPU parity of the microscaling (MXFP8 E4M3) variant against oracle.mx.

* Quantizers: codes and E8M0 scale bytes bit-exact against oracle.mx.quant_mx
  (row blocks) and oracle.mx.quant_mx of the transposed matrix (column
  blocks), for BF16 and FP32 inputs, ragged shapes, special values (all-zero
  blocks, subnormal block maxima, elements that underflow below E4M3's range,
  FP32's largest binade, signed zeros), the dual-output form, and the full
  size of the linear layer's X on sampled rows and columns.
* GEMM: against the float64 contraction of the dequantized operands
  (oracle.mx.gemm_mx_ref), elementwise within the FP8 instruction's bound
  (gpu_util.check_gemm with exact=False).  The scales ride in the matrix
  instruction and the accumulator is chained through it, so up to one FP32
  addition per group of 8 K may round: the bound's FP32 term takes K/8
  additions.  Fprop, Dgrad and Wgrad shapes are built from the MX quantizers'
  outputs, as a training step would call them."""

import numpy as np
import pytest
import torch

import fp8_fine_grained_quant_amd as fq
from oracle import mx
import synth
from gpu_util import DEV, assert_bytes_equal, check_gemm, f32, gpu, log, np_u8, sample_rows

pytestmark = pytest.mark.gpu

DTYPES = pytest.mark.parametrize("dt", [torch.bfloat16, torch.float32], ids=["bf16", "f32"])


def _special(rows, cols, seed):
    """Seeded Student-t data with every special case of the MX rule planted in
    its own 32-block (the first 8 rows)."""
    x = synth.general(rows, cols, seed, kind="t3", outlier_frac=0.01, outlier_mul=50.0)
    if rows >= 8 and cols >= 64:
        x[0, :32] = 0.0                                   # all-zero block: byte 0
        x[0, 32:64] = -0.0                                # signed zeros
        x[1, :32] *= 2.0 ** -125                          # subnormal-range maximum (FP32 input)
        x[2, :32] = 0.0
        x[2, 5] = 2.0 ** 100                              # huge max: every other element ...
        x[2, 6] = -2.0 ** -40                             # ... underflows below E4M3 (-> 0x80)
        x[2, 7] = 2.0 ** 93                               # lands exactly on the grid
        x[3, :32] = 448.0 * 2.0 ** np.arange(-16, 16)     # one binade per element
        x[4, :32] = 3.0e38 * np.linspace(-1, 1, 32)       # FP32's largest binade
        x[5, :32] = 2.0 ** 7 * (1.0 + np.arange(32) / 64)  # max just below a power of two ...
        x[5, 31] = 2.0 ** 8                               # ... then exactly on it
        x[6, :32] = 1.0 + 2.0 ** -4 * np.arange(32)       # ties of the E4M3 grid after scaling
        x[7, :32] = np.linspace(-479.9, 479.9, 32)        # saturating elements
    return x


def _to(x64, dt):
    t = torch.from_numpy(np.asarray(x64, np.float32))
    return t.to(dt) if dt == torch.bfloat16 else t


@DTYPES
@pytest.mark.parametrize("rows,cols", [(1, 32), (37, 208), (300, 1024), (8, 64), (129, 144), (64, 7168)])
def test_quant_mx_rows_bit_exact(rows, cols, dt):
    x = _to(_special(rows, cols, seed=rows * 131 + cols), dt)
    q, s = fq.quant_mx(gpu(x))
    torch.cuda.synchronize()
    rq, rs = mx.quant_mx(f32(x))
    assert_bytes_equal(np_u8(q), rq, f"mx codes {rows}x{cols} {dt}")
    assert_bytes_equal(np_u8(s), rs, f"mx scales {rows}x{cols} {dt}")


@DTYPES
@pytest.mark.parametrize("dual", [False, True], ids=["single", "dual"])
@pytest.mark.parametrize("rows,cols", [(128, 128), (208, 144), (48, 64), (1008, 256), (16, 80)])
def test_quant_mx_transpose_bit_exact(rows, cols, dt, dual):
    x = _to(_special(rows, cols, seed=rows + 977 * cols), dt)
    out = fq.quant_mx_transpose(gpu(x), dual=dual)
    torch.cuda.synchronize()
    xf = f32(x)
    rq_t, rs_t = mx.quant_mx(np.ascontiguousarray(xf.T))
    q_t, s_t = out[-2:]
    assert_bytes_equal(np_u8(q_t), rq_t, f"mx^T codes {rows}x{cols}")
    assert_bytes_equal(np_u8(s_t), rs_t, f"mx^T scales {rows}x{cols}")
    if dual:
        rq, rs = mx.quant_mx(xf)
        assert_bytes_equal(np_u8(out[0]), rq, f"mx dual row codes {rows}x{cols}")
        assert_bytes_equal(np_u8(out[1]), rs, f"mx dual row scales {rows}x{cols}")


def test_quant_mx_strided_outputs_leave_padding():
    rows, cols = 70, 96
    x = gpu(_to(_special(rows, cols, seed=3), torch.bfloat16))
    qb = torch.full((rows, cols + 32), 0xAB, dtype=torch.uint8, device=DEV)
    sb = torch.full((rows, 8), 0xCD, dtype=torch.uint8, device=DEV)
    fq.fp8q_quant_mx_1x32(x, qb[:, :cols], sb[:, :3])
    torch.cuda.synchronize()
    rq, rs = mx.quant_mx(f32(x))
    assert_bytes_equal(np_u8(qb[:, :cols]), rq, "strided codes")
    assert_bytes_equal(np_u8(sb[:, :3]), rs, "strided scales")
    assert torch.all(qb[:, cols:] == 0xAB) and torch.all(sb[:, 3:] == 0xCD)


def test_quant_mx_linear_x_full_size_sampled():
    x, _ = synth.linear_x_w()
    log("C2 X 4096x7168: MX rows and columns, sampled")
    q, s, q_t, s_t = fq.quant_mx_transpose(gpu(x), dual=True)
    q2, s2 = fq.quant_mx(gpu(x))
    torch.cuda.synchronize()
    assert torch.equal(q, q2) and torch.equal(s, s2)
    xf = f32(x)
    rows = sample_rows(4096, 48, 21, must=(0, 4095))
    rq, rs = mx.quant_mx(xf[rows])
    assert_bytes_equal(np_u8(q)[rows], rq, "C2 X mx rows")
    assert_bytes_equal(np_u8(s)[rows], rs, "C2 X mx row scales")
    cols = sample_rows(7168, 48, 22, must=(0, 7167))
    cq, cs = mx.quant_mx(np.ascontiguousarray(xf[:, cols].T))
    assert_bytes_equal(np_u8(q_t)[cols], cq, "C2 X mx columns")
    assert_bytes_equal(np_u8(s_t)[cols], cs, "C2 X mx column scales")


# ---------------------------------------------------------------------- GEMM
def _check_mx(c, aq, as_, bq, bs, out_bf16, what, rows=None):
    """c [M or len(rows), N] from the GPU; the oracle runs on the same codes
    (checked bit-exact against the oracle's quantizer by the tests above)."""
    aq, as_ = np_u8(aq), np_u8(as_)
    if rows is not None:
        aq, as_ = aq[rows], as_[rows]
    k = aq.shape[1]
    y_ref, s_ref = mx.gemm_mx_ref(aq, as_[:, :k // 32], np_u8(bq), np_u8(bs)[:, :k // 32])
    c = f32(c) if torch.is_tensor(c) else c
    return check_gemm(c, y_ref, s_ref, out_bf16, what, exact=False, nk=k // 8)


@pytest.mark.parametrize("m,n,k", [(300, 384, 1024), (1, 128, 128), (257, 256, 384), (512, 128, 2048),
                                   (255, 640, 256), (256, 128, 640)])
@pytest.mark.parametrize("out_dtype", [torch.bfloat16, torch.float32])
def test_gemm_mx_tiles_and_ragged_tail(m, n, k, out_dtype):
    a = _to(synth.general(m, k, seed=m + 3 * k, kind="t3", outlier_frac=0.002, outlier_mul=30.0), torch.bfloat16)
    b = _to(synth.general(n, k, seed=n + 5 * k) * 0.02, torch.float32)
    aq, as_ = fq.quant_mx(gpu(a))
    bq, bs = fq.quant_mx(gpu(b))
    c = fq.gemm_mx(aq, as_, bq, bs, out_dtype=out_dtype)
    torch.cuda.synchronize()
    _check_mx(c, aq, as_, bq, bs, out_dtype == torch.bfloat16, f"mx {m}x{n}x{k}")


@pytest.mark.parametrize("pad", ["word", "block16"])
def test_gemm_mx_padded_scale_rows_and_strided_output(pad):
    """Scale rows padded (pad = 4: 4-byte words, pad to a 16-byte multiple:
    the 4-chunk block loads) and a strided, guarded output."""
    m, n, k = 300, 256, 384
    a = gpu(_to(synth.general(m, k, seed=41, kind="t3"), torch.bfloat16))
    b = gpu(_to(synth.general(n, k, seed=42) * 0.02, torch.float32))
    aq, as0 = fq.quant_mx(a)
    bq, bs0 = fq.quant_mx(b)
    w = k // 32 + 4 if pad == "word" else 16 * ((k // 32 + 15) // 16)
    as_ = torch.full((m, w), 0xEE, dtype=torch.uint8, device=DEV)
    bs = torch.full((n, w), 0xEE, dtype=torch.uint8, device=DEV)
    as_[:, :k // 32] = as0
    bs[:, :k // 32] = bs0
    cbuf = torch.full((m + 1, n + 64), 1234.0, dtype=torch.bfloat16, device=DEV)
    fq.fp8q_gemm_mx(aq, as_, bq, bs, cbuf[:m, :n])
    torch.cuda.synchronize()
    assert torch.all(cbuf[:m, n:] == 1234.0) and torch.all(cbuf[m] == 1234.0)
    _check_mx(cbuf[:m, :n], aq, as0, bq, bs0, True, f"mx padded scales {w}")


def test_gemm_mx_accumulate_and_deterministic():
    m, n, k = 256, 256, 512
    a = gpu(_to(synth.general(m, k, seed=51), torch.bfloat16))
    b = gpu(_to(synth.general(n, k, seed=52), torch.bfloat16))
    aq, as_ = fq.quant_mx(a)
    bq, bs = fq.quant_mx(b)
    c1 = fq.gemm_mx(aq, as_, bq, bs, out_dtype=torch.float32)
    c2 = fq.gemm_mx(aq, as_, bq, bs, out_dtype=torch.float32)
    base = torch.linspace(-3, 3, m * n, device=DEV).reshape(m, n)
    c3 = fq.gemm_mx(aq, as_, bq, bs, c=base.clone())
    torch.cuda.synchronize()
    assert torch.equal(c1, c2)
    assert torch.equal(c3, base + c1)


def test_gemm_mx_training_step_shapes():
    """Fprop, Dgrad and Wgrad of one linear layer in MX, every operand from
    the MX quantizers (rows for Fprop, the transposed blocks for Dgrad's W and
    both Wgrad operands)."""
    t, k, n = 384, 512, 256
    x = gpu(_to(synth.general(t, k, seed=61, outlier_frac=0.02, outlier_mul=20.0), torch.bfloat16))
    w = gpu(_to(synth.general(n, k, seed=62) * 0.02, torch.float32))
    dy = gpu(_to(synth.general(t, n, seed=63, kind="t3"), torch.bfloat16))
    xq, xs, xq_t, xs_t = fq.quant_mx_transpose(x, dual=True)
    wq, ws, wq_t, ws_t = fq.quant_mx_transpose(w, dual=True)
    dyq, dys, dyq_t, dys_t = fq.quant_mx_transpose(dy, dual=True)
    y = fq.gemm_mx(xq, xs, wq, ws)                                   # [t, n]
    dx = fq.gemm_mx(dyq, dys, wq_t, ws_t)                            # [t, k]
    dw = fq.gemm_mx(dyq_t, dys_t, xq_t, xs_t, out_dtype=torch.float32)  # [n, k]
    torch.cuda.synchronize()
    _check_mx(y, xq, xs, wq, ws, True, "mx step fprop")
    _check_mx(dx, dyq, dys, wq_t, ws_t, True, "mx step dgrad")
    _check_mx(dw, dyq_t, dys_t, xq_t, xs_t, False, "mx step wgrad")
    # the operands themselves are the oracle's quantization of the tensors
    assert_bytes_equal(np_u8(wq_t), mx.quant_mx(np.ascontiguousarray(f32(w).T))[0], "W^T mx codes")


def test_gemm_mx_linear_config_full_size_sampled_rows():
    x, w = synth.linear_x_w()
    log("C2 MX fprop 4096x2048x7168, 48 sampled rows")
    xq, xs = fq.quant_mx(gpu(x))
    wq, ws = fq.quant_mx(gpu(w))
    y = fq.gemm_mx(xq, xs, wq, ws)
    torch.cuda.synchronize()
    rows = sample_rows(4096, 48, 23, must=(0, 255, 256, 4095))
    _check_mx(f32(y)[rows], xq, xs, wq, ws, True, "C2 mx fprop", rows=rows)
