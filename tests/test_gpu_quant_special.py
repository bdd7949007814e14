"""Special values through every quantizer, bit-exact against the oracle:
all-zero and signed-zero groups, denormal-only groups below the 2^-100 floor,
max-abs near FLT_MAX (and the BF16 maximum), groups whose maximum only
reaches 448 by saturation after FP32 rounding, E4M3 rounding midpoints,
negative underflow, 2^+-60 magnitudes and one-outlier groups.  Each case runs
on BF16 and FP32 inputs, on a whole-tile shape and on a ragged one.

The rule being checked: each group's max-abs is mapped to the largest E4M3
value (the innerforce.co.kr excerpt of the DeepSeek-V3 report, paragraph on
Figure 7 (a)), applied per 1x128 row group, per 128x128 block and per
128-token column group; underflow and overflow are where FP8 loses
information ("DeepSeek FP8 Training", list of challenges)."""

import numpy as np
import pytest
import torch

import fp8_fine_grained_quant_amd as fq
import oracle
import synth
from gpu_util import assert_bytes_equal, assert_scales_equal, f32, gpu, log, np_u8
from special_values import special_matrix

pytestmark = pytest.mark.gpu

SHAPES = [(384, 13 * 128), (304, 13 * 128 + 48)]  # ragged tails of 48; code rows stay 16-byte multiples
DTYPES = [torch.float32, torch.bfloat16]


def _input(rows, cols, dtype, seed):
    a = special_matrix(rows, cols, seed, for_bf16=dtype == torch.bfloat16)
    return synth.to_bf16(a) if dtype == torch.bfloat16 else torch.from_numpy(a)


def _ids(v):
    return f"{v[0]}x{v[1]}" if isinstance(v, tuple) else str(v).replace("torch.", "")


@pytest.mark.parametrize("shape", SHAPES, ids=_ids)
@pytest.mark.parametrize("dtype", DTYPES, ids=_ids)
def test_special_act_1x128(shape, dtype):
    x_cpu = _input(*shape, dtype, seed=101)
    log(f"special quant_act {shape} {dtype}")
    q, s = fq.quant_act_1x128(gpu(x_cpu))
    torch.cuda.synchronize()
    qo, so = oracle.quant_act_1x128(f32(x_cpu))
    assert_bytes_equal(np_u8(q), qo, "codes")
    assert_scales_equal(s.cpu().numpy(), so, "scales")


@pytest.mark.parametrize("shape", SHAPES, ids=_ids)
@pytest.mark.parametrize("dtype", DTYPES, ids=_ids)
def test_special_weight_128x128_with_transpose(shape, dtype):
    w_cpu = _input(*shape, dtype, seed=102)
    log(f"special quant_weight {shape} {dtype}")
    q, s, q_t = fq.quant_weight_128x128(gpu(w_cpu))
    torch.cuda.synchronize()
    qo, so, qto = oracle.quant_weight_128x128(f32(w_cpu))
    assert_bytes_equal(np_u8(q), qo, "codes")
    assert_scales_equal(s.cpu().numpy(), so, "scales")
    assert_bytes_equal(np_u8(q_t), qto, "transposed codes")


@pytest.mark.parametrize("shape", SHAPES, ids=_ids)
@pytest.mark.parametrize("dtype", DTYPES, ids=_ids)
def test_special_transpose(shape, dtype):
    x_cpu = _input(*shape, dtype, seed=103)
    log(f"special quant_transpose {shape} {dtype}")
    q_t, s_t = fq.quant_transpose(gpu(x_cpu))
    torch.cuda.synchronize()
    qo, so = oracle.quant_transpose(f32(x_cpu))
    assert_bytes_equal(np_u8(q_t), qo, "codes")
    assert_scales_equal(s_t.cpu().numpy(), so, "scales")


@pytest.mark.parametrize("shape", SHAPES, ids=_ids)
@pytest.mark.parametrize("dtype", DTYPES, ids=_ids)
def test_special_act_transpose(shape, dtype):
    x_cpu = _input(*shape, dtype, seed=104)
    log(f"special quant_act_transpose {shape} {dtype}")
    q, s, q_t, s_t = fq.quant_act_transpose(gpu(x_cpu))
    torch.cuda.synchronize()
    qo, so = oracle.quant_act_1x128(f32(x_cpu))
    qto, sto = oracle.quant_transpose(f32(x_cpu))
    assert_bytes_equal(np_u8(q), qo, "row codes")
    assert_scales_equal(s.cpu().numpy(), so, "row scales")
    assert_bytes_equal(np_u8(q_t), qto, "transposed codes")
    assert_scales_equal(s_t.cpu().numpy(), sto, "transposed scales")


@pytest.mark.parametrize("counts", [[5, 0, 295, 1, 130, 128, 0, 200], [384], [127, 257]],
                         ids=["ragged", "one", "two"])
@pytest.mark.parametrize("cols", [13 * 128, 200])
@pytest.mark.parametrize("dtype", DTYPES, ids=_ids)
def test_special_transpose_grouped(counts, cols, dtype):
    m = int(sum(counts))
    x_cpu = _input(m, cols, dtype, seed=105 + m + cols)
    off = torch.tensor(np.concatenate([[0], np.cumsum(counts)]), dtype=torch.int32)
    log(f"special quant_transpose_grouped {counts} cols={cols} {dtype}")
    q_t, s_t = fq.quant_transpose_grouped(gpu(x_cpu), gpu(off))
    torch.cuda.synchronize()
    qo, so, col_def, chunk_def = oracle.quant_transpose_grouped(f32(x_cpu), off.numpy())
    assert_bytes_equal(np_u8(q_t)[:, col_def], qo[:, col_def], "codes")
    assert_scales_equal(f32(s_t)[:, chunk_def], so[:, chunk_def], "scales")
    # the padding of each expert's last chunk is code 0
    assert not np_u8(q_t)[:, ~col_def].any()
