"""Microscaling (MX) variant of the oracle (test infrastructure only).

The pages contrast the method's FP32 group scales with microscaling formats
that hardware supports natively (the innerforce.co.kr excerpt, paragraph on
Figure 7 (a): small groups with power-of-two scales, as in NVIDIA's
Blackwell microscaling formats).  This variant follows the OCP Microscaling
(MX) v1.0 definition of MXFP8 with E4M3 elements:

* a block is 32 consecutive elements along the contraction axis, for both
  GEMM operands (activations and weights alike);
* the shared scale is the power of two X = 2^(floor(log2 amax) - 8), 8 being
  the exponent of E4M3's largest power of two (256), stored as an E8M0 byte
  e + 127 (clamped to [0, 254]); an all-zero block takes the smallest scale,
  byte 0;
* each element is encode(x / X): E4M3 with round-to-nearest-even and
  saturation to +-448 (x / X lies in [256, 512) for the block's largest
  element, so values above 448 saturate).

The GEMM result is the exact contraction of the dequantized operands, as for
the method; the kernel's scaled matrix instruction applies the block scales
itself and accumulates in FP32.
"""

import numpy as np

from .e4m3 import decode, encode

BLOCK = 32


def e8m0_of_amax(amax):
    """amax (float array) -> E8M0 scale bytes (uint8): floor(log2 amax) - 8 + 127,
    clamped to [0, 254]; amax == 0 gives 0."""
    amax = np.asarray(amax, dtype=np.float64)
    out = np.zeros(amax.shape, dtype=np.int64)
    nz = amax > 0
    _, ex = np.frexp(amax[nz])                     # amax = m * 2^ex with m in [0.5, 1)
    out[nz] = np.clip(ex - 1 - 8 + 127, 0, 254)    # floor(log2 amax) = ex - 1
    return out.astype(np.uint8)


def scale_value(byte):
    """E8M0 byte -> its power of two (float64)."""
    return np.ldexp(1.0, np.asarray(byte, dtype=np.int64) - 127)


def quant_mx(x):
    """x float32 [R, C] -> (q uint8 [R, C], s uint8 [R, ceil(C/32)]): MXFP8
    E4M3 along the rows (blocks of 32 consecutive columns; a trailing partial
    block uses the elements present)."""
    x = np.asarray(x, dtype=np.float32)
    rows, cols = x.shape
    nb = (cols + BLOCK - 1) // BLOCK
    q = np.zeros((rows, cols), dtype=np.uint8)
    s = np.zeros((rows, nb), dtype=np.uint8)
    for j in range(nb):
        blk = x[:, j * BLOCK:(j + 1) * BLOCK].astype(np.float64)
        sb = e8m0_of_amax(np.abs(blk).max(axis=1) if rows else np.zeros(0))
        # x / X is exact in float64 (X is a power of two, no underflow for
        # float32 inputs); encode rounds it once, to nearest even
        q[:, j * BLOCK:(j + 1) * BLOCK] = encode(blk / scale_value(sb)[:, None])
        s[:, j] = sb
    return q, s


def dequant_mx(q, s):
    q = np.asarray(q)
    idx = np.arange(q.shape[1]) // BLOCK
    return decode(q) * scale_value(np.asarray(s))[:, idx]


def gemm_mx_ref(aq, as_, bq, bs):
    """C[M,N] = A . B^T of the dequantized MX operands (both blocked along K).
    Returns (C, S) float64 with S = sum_k |a b|."""
    a = dequant_mx(aq, as_)
    b = dequant_mx(bq, bs)
    return a @ b.T, np.abs(a) @ np.abs(b).T
