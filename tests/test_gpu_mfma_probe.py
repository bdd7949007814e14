"""Accumulation precision of gfx950's FP8 matrix instruction, measured through
the GEMM entry points (the counterpart of the H800 Tensor Core measurement in
the innerforce.co.kr excerpt, paragraph after Figure 7 (a), which finds about
14 bits kept there).

Probe: one 128-K chunk, all scales 1, two non-zero products per output
(codes are exact powers of two, so every product is exact in FP32): a large
one 2^e and a small one 2^(e-t).
  * Both in the same group of 8 consecutive K: the FP8 entry point keeps the
    small product while t <= 13 and drops it (truncation) from t = 14 on,
    i.e. 14 bits below and including the largest product's leading bit.
  * In different groups of 8: the groups are summed in FP32, so the small
    product survives until FP32's own 24-bit precision.
  * The exact-accumulation entry point keeps it in both cases.
These are the facts the FP8 tolerance bound of the parity tests rests on."""

import numpy as np
import pytest
import torch

import fp8_fine_grained_quant_amd as fq
from gpu_util import DEV, log

pytestmark = pytest.mark.gpu

M, N, K = 16, 128, 128


def _code_pow2(e):
    """E4M3 code of +2^e for -9 <= e <= 8 (subnormals below -6)."""
    if e < -6:
        return 1 << (e + 9)            # subnormal: F * 2^-9 with F = 2^(e+9)
    return (e + 7) << 3


def _probe(k_small, gap, exact):
    """Output[0, 0] of a one-chunk GEMM with products 2^6 * 2^6 at K = 0 and
    2^(12 - gap) at K = k_small; returns (got, exact value)."""
    a = torch.zeros(M, K, dtype=torch.uint8)
    b = torch.zeros(N, K, dtype=torch.uint8)
    a[0, 0] = _code_pow2(6)
    b[0, 0] = _code_pow2(6)
    ea = min(8, max(-9, 12 - gap - 8))
    eb = 12 - gap - ea
    assert -9 <= ea <= 8 and -9 <= eb <= 8, (gap, ea, eb)
    a[0, k_small] = _code_pow2(ea)
    b[0, k_small] = _code_pow2(eb)
    xs = torch.ones(M, K // 128)
    ws = torch.ones(N // 128, K // 128)
    y = fq.gemm_fprop(a.to(DEV), xs.to(DEV), b.to(DEV), ws.to(DEV), out_dtype=torch.float32, exact=exact)
    torch.cuda.synchronize()
    return float(y[0, 0]), 2.0 ** 12 + 2.0 ** (12 - gap)


def _survives(k_small, gap, exact):
    got, want = _probe(k_small, gap, exact)
    assert got in (2.0 ** 12, want), (k_small, gap, got)
    return got == want


def test_fp8_instruction_keeps_14_bits_within_a_group_of_8():
    kept = [g for g in range(1, 24) if _survives(1, g, exact=False)]
    log(f"same group of 8: small product kept at gaps {kept}")
    assert kept == list(range(1, 14)), kept


def test_groups_of_8_are_summed_in_fp32():
    kept = [g for g in range(1, 24) if _survives(8, g, exact=False)]
    log(f"next group of 8: small product kept at gaps {kept}")
    assert kept == list(range(1, 24)), kept
    # the group boundary is at K = 8: position 7 is still in the first group
    assert not _survives(7, 16, exact=False)


def test_exact_entry_point_keeps_every_product():
    for k_small in (1, 7, 8):
        kept = [g for g in range(1, 24) if _survives(k_small, g, exact=True)]
        assert kept == list(range(1, 24)), (k_small, kept)
