"""GPU parity of the MoE backward products against the oracle: the grouped
quantize-transpose (bit-exact codes and scales, zero padding), grouped Dgrad
and grouped Wgrad (the FP8 matrix-instruction bound of gpu_util.check_gemm),
plus bit-identity with the dense entry points applied expert by expert."""

import numpy as np
import pytest
import torch

import fp8_fine_grained_quant_amd as fq
import oracle
import synth
from gpu_util import DEV, assert_bytes_equal, assert_scales_equal, check_gemm, f32, gpu, log, np_u8, sample_rows

pytestmark = pytest.mark.gpu


def _offsets(counts):
    return torch.tensor(np.concatenate([[0], np.cumsum(counts)]), dtype=torch.int32)


RAGGED = [
    [5, 0, 295, 1, 399, 128, 0, 130],
    [128, 256, 0, 384],
    [1],
    [0, 0, 700],
    [127, 129, 255, 257, 0, 3],
]


# ------------------------------------------------------ grouped quantize-transpose
def _check_transpose_grouped(x_cpu, counts, what):
    off = _offsets(counts)
    q_t, s_t = fq.quant_transpose_grouped(gpu(x_cpu), gpu(off))
    torch.cuda.synchronize()
    qo, so, col_def, chunk_def = oracle.quant_transpose_grouped(f32(x_cpu), off.numpy())
    assert q_t.shape == qo.shape and s_t.shape == so.shape
    assert_bytes_equal(np_u8(q_t)[:, col_def], qo[:, col_def], what + " codes")
    assert_scales_equal(f32(s_t)[:, chunk_def], so[:, chunk_def], what + " scales")


@pytest.mark.parametrize("counts", RAGGED, ids=[f"case{i}" for i in range(len(RAGGED))])
@pytest.mark.parametrize("cols,dtype", [(256, torch.bfloat16), (384, torch.float32), (200, torch.float32),
                                        (24, torch.bfloat16)])
def test_quant_transpose_grouped_small(counts, cols, dtype):
    m = int(sum(counts))
    x = synth.general(m, cols, seed=m + cols, kind="t3", outlier_frac=0.01, outlier_mul=50.0)
    x_cpu = synth.to_bf16(x) if dtype == torch.bfloat16 else torch.from_numpy(x.astype(np.float32))
    log(f"quant_transpose_grouped counts={counts} cols={cols} {dtype}")
    _check_transpose_grouped(x_cpu, counts, f"grouped transpose {counts} {cols}")


def test_quant_transpose_grouped_moe_dy_full():
    dy = synth.moe_dy()
    _, _, offsets = _moe()
    log("C6 dY [16384,2048] grouped transpose, all channels")
    _check_transpose_grouped(dy, np.diff(offsets.numpy()).tolist(), "C6 dY")


def test_quant_transpose_grouped_moe_x_channel_sample():
    x, _, offsets = _moe()
    chans = np.sort(np.random.Generator(np.random.PCG64(31)).choice(7168, size=256, replace=False))
    log("C5 X [16384,7168] grouped transpose, 256 sampled channels")
    off = gpu(offsets)
    q_t, s_t = fq.quant_transpose_grouped(gpu(x), off)
    torch.cuda.synchronize()
    qo, so, col_def, chunk_def = oracle.quant_transpose_grouped(f32(x[:, torch.from_numpy(chans)]),
                                                                offsets.numpy())
    assert_bytes_equal(np_u8(q_t)[chans][:, col_def], qo[:, col_def], "C5 X codes")
    assert_scales_equal(f32(s_t)[chans][:, chunk_def], so[:, chunk_def], "C5 X scales")


_MOE = {}


def _moe():
    if "v" not in _MOE:
        _MOE["v"] = synth.moe_fprop()
    return _MOE["v"]


# ---------------------------------------------------------------- grouped Dgrad
def _dgrad_case(counts, n, k, seed, out_dtype=torch.bfloat16):
    off = _offsets(counts)
    m = int(off[-1])
    e = len(counts)
    rng = np.random.Generator(np.random.PCG64(seed))
    dy_cpu = synth.to_bf16(rng.standard_t(3, size=(m, n)))
    w_cpu = torch.from_numpy((rng.standard_normal((e * n, k)) * 0.02).astype(np.float32))
    dyq, dys = fq.quant_act_1x128(gpu(dy_cpu))
    wq, ws, wq_t = fq.quant_weight_128x128(gpu(w_cpu), transpose=True)
    dx = fq.grouped_gemm_dgrad(dyq, dys, wq_t, ws, gpu(off), out_dtype=out_dtype)
    torch.cuda.synchronize()
    return off, dy_cpu, w_cpu, (dyq, dys, wq, ws, wq_t), dx


@pytest.mark.parametrize("counts,n,k", [([5, 0, 295, 1, 399], 256, 384), ([300], 128, 256),
                                        ([0, 1000, 0], 384, 128), ([127, 129, 256, 0, 3], 128, 512)])
@pytest.mark.parametrize("out_dtype", [torch.bfloat16, torch.float32])
def test_grouped_dgrad_small_all_rows(counts, n, k, out_dtype):
    log(f"grouped dgrad counts={counts} n={n} k={k} {out_dtype}")
    off, dy_cpu, w_cpu, _, dx = _dgrad_case(counts, n, k, seed=sum(counts) + n + k, out_dtype=out_dtype)
    dyo, dyso = oracle.quant_act_1x128(f32(dy_cpu))
    wo, wso, wo_t = oracle.quant_weight_128x128(f32(w_cpu))
    y_ref, s_ref = oracle.grouped_dgrad_ref(dyo, dyso, wo_t, wso, off.numpy())
    check_gemm(f32(dx), y_ref, s_ref, out_dtype == torch.bfloat16, f"grouped dgrad {counts}", False, nk=n // 128)


def test_grouped_dgrad_equals_per_expert_dgrad():
    counts, n, k = [70, 0, 300, 1, 258], 256, 384
    off, _, _, (dyq, dys, wq, ws, wq_t), dx = _dgrad_case(counts, n, k, seed=3)
    o = off.tolist()
    for i in range(len(counts)):
        lo, hi = o[i], o[i + 1]
        if hi == lo:
            continue
        w_t = wq_t[:, i * n:(i + 1) * n].contiguous()
        de = fq.gemm_dgrad(dyq[lo:hi], dys[lo:hi], w_t, ws[i * n // 128:(i + 1) * n // 128].contiguous())
        assert torch.equal(de, dx[lo:hi]), f"expert {i}"


@pytest.mark.timeout(600)
def test_grouped_dgrad_moe_config_sampled_rows():
    x, w, offsets = _moe()
    e, n, k = w.shape
    dy = synth.moe_dy()
    log(f"C6 grouped dgrad: dY [16384,2048] . W_e, 32 experts, counts {np.diff(offsets.numpy()).tolist()}")
    dyq, dys = fq.quant_act_1x128(gpu(dy))
    wq, ws, wq_t = fq.quant_weight_128x128(gpu(w.reshape(e * n, k)), transpose=True)
    dx = fq.grouped_gemm_dgrad(dyq, dys, wq_t, ws, gpu(offsets))
    torch.cuda.synchronize()
    off = offsets.numpy().astype(np.int64)
    rows = sample_rows(int(off[-1]), 48, 41, must=tuple(int(v) for v in off[1:-1] if v < off[-1]))
    experts = np.searchsorted(off, rows, side="right") - 1
    dyo, dyso = oracle.quant_act_1x128(f32(dy[torch.from_numpy(rows)]))
    y_ref = np.zeros((rows.size, k))
    s_ref = np.zeros((rows.size, k))
    for ex in np.unique(experts):
        wo, wso, _ = oracle.quant_weight_128x128(f32(w[int(ex)]))
        sel = np.nonzero(experts == ex)[0]
        y_ref[sel], s_ref[sel] = oracle.dgrad_ref(dyo[sel], dyso[sel], wo, wso)
    check_gemm(f32(dx)[rows], y_ref, s_ref, True, "C6 grouped dgrad", False, nk=n // 128, strict=True)


# ---------------------------------------------------------------- grouped Wgrad
def _wgrad_case(counts, n, k, seed):
    off = _offsets(counts)
    m = int(off[-1])
    rng = np.random.Generator(np.random.PCG64(seed))
    x_cpu = synth.to_bf16(rng.standard_normal((m, k)) * rng.choice([1.0, 20.0], size=(1, k), p=[0.98, 0.02]))
    dy_cpu = synth.to_bf16(rng.standard_t(3, size=(m, n)))
    og = gpu(off)
    xq_t, xs_t = fq.quant_transpose_grouped(gpu(x_cpu), og)
    dyq_t, dys_t = fq.quant_transpose_grouped(gpu(dy_cpu), og)
    dw = fq.grouped_gemm_wgrad(dyq_t, dys_t, xq_t, xs_t, og, m)
    torch.cuda.synchronize()
    return off, x_cpu, dy_cpu, (dyq_t, dys_t, xq_t, xs_t), dw


@pytest.mark.parametrize("counts,n,k", [([5, 0, 295, 1, 399], 256, 384), ([300], 128, 256),
                                        ([0, 1000, 0], 104, 128), ([127, 129, 256, 0, 3], 296, 256)])
def test_grouped_wgrad_small_all_outputs(counts, n, k):
    log(f"grouped wgrad counts={counts} n={n} k={k}")
    off, x_cpu, dy_cpu, _, dw = _wgrad_case(counts, n, k, seed=sum(counts) + n + k)
    gx = oracle.quant_transpose_grouped(f32(x_cpu), off.numpy())
    gdy = oracle.quant_transpose_grouped(f32(dy_cpu), off.numpy())
    y_ref, s_ref = oracle.grouped_wgrad_ref(gdy[0], gdy[1], gx[0], gx[1], off.numpy())
    nk = max(1, max(-(-c // 128) for c in counts))
    check_gemm(f32(dw).reshape(-1, k), y_ref.reshape(-1, k), s_ref.reshape(-1, k), False,
               f"grouped wgrad {counts}", False, nk=nk)


def test_grouped_wgrad_equals_per_expert_dense_wgrad_and_accumulates():
    counts, n, k = [130, 0, 1, 300, 256], 256, 384
    off, _, _, (dyq_t, dys_t, xq_t, xs_t), dw = _wgrad_case(counts, n, k, seed=5)
    p = oracle.padded_starts(off.numpy())
    for i, m in enumerate(counts):
        if m == 0:
            assert torch.all(dw[i] == 0), f"expert {i} has no tokens"
            continue
        nc = -(-m // 128)
        c0, c1 = int(p[i]), int(p[i]) + 128 * nc
        de = fq.gemm_wgrad(dyq_t[:, c0:c1].contiguous(), dys_t[:, c0 // 128:c1 // 128].contiguous(),
                           xq_t[:, c0:c1].contiguous(), xs_t[:, c0 // 128:c1 // 128].contiguous())
        assert torch.equal(de, dw[i]), f"expert {i}"
    # accumulate: dW += the same product; an empty expert keeps its contents
    acc = torch.full_like(dw, 0.5)
    fq.grouped_gemm_wgrad(dyq_t, dys_t, xq_t, xs_t, gpu(off), int(off[-1]), dw=acc)
    torch.cuda.synchronize()
    assert torch.all(acc[1] == 0.5)
    assert torch.allclose(acc, dw + 0.5, rtol=2 ** -22, atol=2 ** -22)


@pytest.mark.timeout(600)
def test_grouped_wgrad_moe_config_sampled_outputs():
    x, w, offsets = _moe()
    n, k = 2048, 7168
    dy = synth.moe_dy()
    og = gpu(offsets)
    m = int(offsets[-1])
    log("C5/C6 grouped wgrad: dW_e = dY_e^T X_e, 32 experts [2048,7168]")
    xq_t, xs_t = fq.quant_transpose_grouped(gpu(x), og)
    dyq_t, dys_t = fq.quant_transpose_grouped(gpu(dy), og)
    dw = fq.grouped_gemm_wgrad(dyq_t, dys_t, xq_t, xs_t, og, m)
    torch.cuda.synchronize()
    off = offsets.numpy().astype(np.int64)
    counts = np.diff(off)
    rng = np.random.Generator(np.random.PCG64(43))
    experts = [int(np.argmax(counts)), int(np.argmin(np.where(counts > 0, counts, 1 << 30)))] + \
        rng.choice(np.nonzero(counts)[0], size=2, replace=False).tolist()
    for e in experts:
        for i in np.nonzero(counts == 0)[0]:
            assert torch.all(dw[int(i)] == 0)
        lo, hi = int(off[e]), int(off[e + 1])
        nr = np.sort(rng.choice(n, size=8, replace=False))
        kc = np.sort(rng.choice(k, size=96, replace=False))
        dyo_t, dyso_t = oracle.quant_transpose(f32(dy[lo:hi][:, torch.from_numpy(nr)]))
        xo_t, xso_t = oracle.quant_transpose(f32(x[lo:hi][:, torch.from_numpy(kc)]))
        y_ref, s_ref = oracle.wgrad_ref(dyo_t, dyso_t, xo_t, xso_t)
        got = f32(dw[e])[nr][:, kc]
        check_gemm(got, y_ref, s_ref, False, f"C5/C6 grouped wgrad expert {e} ({hi - lo} tokens)", False,
                   nk=-(-(hi - lo) // 128))
