"""Seeded random shapes through the microscaling variant: the row, transposing
and dual MX quantizers bit-exact against oracle.mx (on inputs with every
special case of the MX rule planted, BF16 and FP32), and the MX GEMM against
oracle.mx.gemm_mx_ref at the bar of test_gpu_mx.py, with a random output type
and workgroup tile.  Shapes come from a counter-based generator per case."""

import numpy as np
import pytest
import torch

import fp8_fine_grained_quant_amd as fq
from oracle import mx
import synth
from gpu_util import assert_bytes_equal, f32, gpu, log, np_u8
from test_gpu_mx import _check_mx, _special, _to

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("case", range(48))
def test_mx_shape_sweep(case):
    rng = np.random.Generator(np.random.PCG64(31000 + case))
    dt = torch.bfloat16 if rng.random() < 0.5 else torch.float32
    rows = int(rng.integers(1, 40)) * 16  # codes need 16-byte row strides, both layouts
    cols = int(rng.integers(1, 70)) * 16
    log(f"mx case {case}: quantizers {rows}x{cols} {dt}")
    x = _to(_special(rows, cols, seed=case), dt)
    q, s = fq.quant_mx(gpu(x))
    dq, ds, dq_t, ds_t = fq.quant_mx_transpose(gpu(x), dual=True)
    torch.cuda.synchronize()
    xf = f32(x)
    rq, rs = mx.quant_mx(xf)
    rq_t, rs_t = mx.quant_mx(np.ascontiguousarray(xf.T))
    assert_bytes_equal(np_u8(q), rq, "mx row codes")
    assert_bytes_equal(np_u8(s), rs, "mx row scales")
    assert_bytes_equal(np_u8(dq), rq, "mx dual row codes")
    assert_bytes_equal(np_u8(ds), rs, "mx dual row scales")
    assert_bytes_equal(np_u8(dq_t), rq_t, "mx transposed codes")
    assert_bytes_equal(np_u8(ds_t), rs_t, "mx transposed scales")

    m = int(rng.integers(1, 700))
    n = int(rng.integers(1, 8)) * 128
    k = int(rng.integers(1, 15)) * 128
    out_dtype = torch.bfloat16 if rng.random() < 0.5 else torch.float32
    tile = str(rng.choice(["auto", "256x128", "256x256"]))
    log(f"mx case {case}: gemm {m}x{n}x{k} {out_dtype} tile={tile}")
    a = _to(synth.general(m, k, seed=case + 7, kind="t3", outlier_frac=0.002, outlier_mul=30.0), torch.bfloat16)
    b = _to(synth.general(n, k, seed=case + 8) * 0.02, torch.float32)
    aq, as_ = fq.quant_mx(gpu(a))
    bq, bs = fq.quant_mx(gpu(b))
    fq.set_gemm_tile(tile)
    try:
        c = fq.gemm_mx(aq, as_, bq, bs, out_dtype=out_dtype)
        torch.cuda.synchronize()
    finally:
        fq.set_gemm_tile("auto")
    _check_mx(c, aq, as_, bq, bs, out_dtype == torch.bfloat16, f"mx sweep {m}x{n}x{k} {tile}")
