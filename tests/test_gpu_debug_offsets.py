"""The FP8Q_DEBUG build (libfp8q_debug.so) of every grouped entry point:
with well-formed expert offsets it gives the product library's result bit for
bit; with malformed ones (offsets[0] != 0, a decrease, offsets[E] != M_total)
it returns FP8Q_ERR_SHAPE and leaves the output untouched.  The malformed
offsets never reach a kernel: the check runs on the host before any launch."""

import numpy as np
import pytest
import torch

import fp8_fine_grained_quant_amd as fq
import synth
from gpu_util import gpu, log

pytestmark = pytest.mark.gpu

COUNTS = [100, 0, 300, 50]          # one empty expert, ragged tails
E, M, N, K = len(COUNTS), sum(COUNTS), 256, 256
SHAPE = 2


def _offsets(vals):
    return gpu(torch.tensor(vals, dtype=torch.int32))


GOOD = list(np.concatenate([[0], np.cumsum(COUNTS)]))
BAD = {
    "first_not_zero": [1] + GOOD[1:],
    "decreasing": [0, 100, 50, 400, M],
    "last_not_total": GOOD[:-1] + [M - 1],
}


def _operands():
    x = synth.to_bf16(synth.general(M, K, seed=11, kind="t3"))
    dy = synth.to_bf16(synth.general(M, N, seed=12, kind="normal"))
    w = torch.from_numpy((synth.general(E * N, K, seed=13) * 0.02).astype(np.float32))
    return gpu(x), gpu(dy), gpu(w)


def _calls(x, dy, w):
    """Each grouped entry point as (name, fn(offsets) -> output tensor)."""
    xq, xs = fq.quant_act_1x128(x)
    dyq, dys = fq.quant_act_1x128(dy)
    wq, ws, wq_t = fq.quant_weight_128x128(w)
    wq3, ws3 = wq.reshape(E, N, K), ws.reshape(E, N // 128, K // 128)
    xmq, xms = fq.quant_mx(x)
    dymq, dyms = fq.quant_mx(dy)
    wmq, wms = fq.quant_mx(w)
    wmq_t, wms_t = fq.quant_mx_transpose(w)
    good = _offsets(GOOD)
    xq_t, xs_t = fq.quant_transpose_grouped(x, good)
    dq_t, ds_t = fq.quant_transpose_grouped(dy, good)
    torch.cuda.synchronize()

    def transpose_grouped(off):
        cap = fq.token_capacity(M, E)
        q_t = torch.full((K, cap), 0x5A, dtype=torch.uint8, device=x.device)
        s_t = torch.full((K, cap // 128), -1.0, dtype=torch.float32, device=x.device)
        fq.fp8q_quant_transpose_grouped(x, off, q_t, s_t)
        return torch.cat([q_t.flatten(), s_t.flatten().view(torch.uint8)])

    def filled(shape, dtype):
        return torch.full(shape, -7.0, dtype=dtype, device=x.device)

    def fprop(exact):
        def run(off):
            y = filled((M, N), torch.bfloat16)
            fq.fp8q_grouped_gemm(xq, xs, wq3, ws3, off, y, exact=exact)
            return y
        return run

    def dgrad(off):
        dx = filled((M, K), torch.bfloat16)
        fq.fp8q_grouped_gemm_dgrad(dyq, dys, wq_t, ws, off, dx)
        return dx

    def wgrad(off):
        dw = filled((E, N, K), torch.float32)
        fq.fp8q_grouped_gemm_wgrad(dq_t, ds_t, xq_t, xs_t, off, M, dw, False)
        return dw

    def mx_fprop(off):
        y = filled((M, N), torch.bfloat16)
        fq.fp8q_grouped_gemm_mx(xmq, xms, wmq.reshape(E, N, K), wms.reshape(E, N, K // 32), off, y)
        return y

    def mx_dgrad(off):
        dx = filled((M, K), torch.bfloat16)
        fq.fp8q_grouped_gemm_mx_dgrad(dymq, dyms, wmq_t, wms_t, off, dx)
        return dx

    return [("quant_transpose_grouped", transpose_grouped), ("grouped_gemm", fprop(False)),
            ("grouped_gemm_exact", fprop(True)), ("grouped_gemm_dgrad", dgrad),
            ("grouped_gemm_wgrad", wgrad), ("grouped_gemm_mx", mx_fprop), ("grouped_gemm_mx_dgrad", mx_dgrad)]


def test_debug_build_checks_offsets(monkeypatch):
    x, dy, w = _operands()
    calls = _calls(x, dy, w)
    product = {}
    for name, fn in calls:
        product[name] = fn(_offsets(GOOD)).clone()
    torch.cuda.synchronize()

    monkeypatch.setattr(fq, "load_library", fq.load_debug_library)
    for name, fn in calls:
        log(f"debug build, well-formed offsets: {name}")
        out = fn(_offsets(GOOD))
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.uint8), product[name].view(torch.uint8)), name
        for case, vals in BAD.items():
            log(f"debug build, {case}: {name}")
            off = _offsets(vals)
            with pytest.raises(fq.Fp8qError) as err:
                fn(off)
            assert err.value.status == SHAPE, (name, case)
    torch.cuda.synchronize()


def test_debug_build_leaves_output_untouched():
    """A rejected call enqueues nothing: the output keeps its fill."""
    x, dy, w = _operands()
    xq, xs = fq.quant_act_1x128(x)
    wq, ws, _ = fq.quant_weight_128x128(w)
    y = torch.full((M, N), -7.0, dtype=torch.bfloat16, device=x.device)
    lib = fq.load_debug_library()
    off = _offsets(BAD["decreasing"])
    st = lib.fp8q_grouped_gemm(xq.data_ptr(), xs.data_ptr(), wq.data_ptr(), ws.data_ptr(), off.data_ptr(), E, M, N,
                               K, y.data_ptr(), 0, N, None)
    torch.cuda.synchronize()
    assert st == SHAPE
    assert bool((y == -7.0).all())
