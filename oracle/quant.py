"""Fine-grained online quantizers of the oracle (test infrastructure only).

Rule for one group (the innerforce.co.kr excerpt of the DeepSeek-V3 report,
paragraph on Figure 7 (a): the group's max-abs is mapped to the largest FP8
value; "unified E4M3 format" page, section "Dynamic Scaling and Online
Quantization": the scale comes from the group's current values):

    amax  = max |x| over the group          (exact)
    amax' = max(amax, 2^-100)               (reading: avoids 0/0 for zero groups)
    s     = fl32(amax' / 448)               (the stored FP32 scale)
    inv   = fl32(448 / amax')
    q     = encode(fl32(x * inv))           (E4M3, RNE, saturating)

All arithmetic is IEEE float32 with round-to-nearest-even, as numpy performs
it on float32 arrays.  The inputs are float32 arrays; BF16 inputs are widened
to float32 first, which is exact.

Groupings:
* quant_act_1x128      -- 1x128 tiles: one token (row), 128 channels (columns);
                          same page and paragraph, item (1).
* quant_weight_128x128 -- 128x128 blocks of rows x columns; item (2).
* quant_transpose      -- the 1x128 rule applied to the transposed matrix:
                          groups are 128 consecutive tokens of one channel and
                          the codes are written transposed (operands of the
                          weight-gradient GEMM, "DeepSeek FP8 Training",
                          weight-gradient list; the grouping axis is a reading).
A trailing partial group uses only the elements that exist.
"""

import numpy as np

from .e4m3 import encode

GROUP = 128
AMAX_FLOOR = np.float32(2.0 ** -100)
FP8_MAX = np.float32(448.0)


def group_scale(amax):
    """amax (float32 array) -> (s, inv), both float32, per the rule above."""
    amax = np.asarray(amax, dtype=np.float32)
    amax_p = np.maximum(amax, AMAX_FLOOR)
    s = np.divide(amax_p, FP8_MAX, dtype=np.float32)
    inv = np.divide(FP8_MAX, amax_p, dtype=np.float32)
    return s, inv


def _ngroups(n):
    return (n + GROUP - 1) // GROUP


def quant_act_1x128(x):
    """x float32 [R, C] -> (q uint8 [R, C], s float32 [R, ceil(C/128)])."""
    x = np.asarray(x, dtype=np.float32)
    rows, cols = x.shape
    g = _ngroups(cols)
    q = np.zeros((rows, cols), dtype=np.uint8)
    s = np.zeros((rows, g), dtype=np.float32)
    for j in range(g):
        blk = x[:, j * GROUP:(j + 1) * GROUP]
        amax = np.abs(blk).max(axis=1) if rows else np.zeros(0, np.float32)
        sj, inv = group_scale(amax)
        y = np.multiply(blk, inv[:, None], dtype=np.float32)
        q[:, j * GROUP:(j + 1) * GROUP] = encode(y)
        s[:, j] = sj
    return q, s


def quant_weight_128x128(w):
    """w float32 [R, C] -> (q uint8 [R, C], s float32 [ceil(R/128), ceil(C/128)],
    q_t uint8 [C, R]).  q_t is q transposed byte for byte: a block's scale does
    not change when the block is transposed."""
    w = np.asarray(w, dtype=np.float32)
    rows, cols = w.shape
    gi, gj = _ngroups(rows), _ngroups(cols)
    q = np.zeros((rows, cols), dtype=np.uint8)
    s = np.zeros((gi, gj), dtype=np.float32)
    for i in range(gi):
        for j in range(gj):
            blk = w[i * GROUP:(i + 1) * GROUP, j * GROUP:(j + 1) * GROUP]
            sij, inv = group_scale(np.abs(blk).max())
            q[i * GROUP:(i + 1) * GROUP, j * GROUP:(j + 1) * GROUP] = encode(
                np.multiply(blk, inv, dtype=np.float32))
            s[i, j] = sij
    return q, s, np.ascontiguousarray(q.T)


def quant_transpose(x):
    """x float32 [R tokens, C channels] -> (q_t uint8 [C, R], s_t float32
    [C, ceil(R/128)]): groups are x[128i:128i+128, c]; q_t[c, r] is the code
    of x[r, c]."""
    x = np.asarray(x, dtype=np.float32)
    rows, cols = x.shape
    g = _ngroups(rows)
    q_t = np.zeros((cols, rows), dtype=np.uint8)
    s_t = np.zeros((cols, g), dtype=np.float32)
    for i in range(g):
        blk = x[i * GROUP:(i + 1) * GROUP, :]           # [<=128 tokens, C]
        amax = np.abs(blk).max(axis=0) if cols else np.zeros(0, np.float32)
        si, inv = group_scale(amax)                     # one per channel
        y = np.multiply(blk, inv[None, :], dtype=np.float32)
        q_t[:, i * GROUP:(i + 1) * GROUP] = encode(y).T
        s_t[:, i] = si
    return q_t, s_t
