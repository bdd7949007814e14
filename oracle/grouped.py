"""Grouped (MoE) backward products of the oracle (test infrastructure only).

The MoE layers of the method run their GEMMs in FP8 like the dense ones (the
innerforce.co.kr excerpt of the DeepSeek-V3 report, the FP8 framework
paragraph: the FP8 GEMMs of linear and MoE layers), with the same operands per
product as the dense layer ("DeepSeek FP8 Training", the weight-gradient and
input-gradient lists).  Per expert e with tokens [o_e, o_{e+1}):

    grouped Dgrad  dX[o_e:o_{e+1}] = dY[o_e:o_{e+1}] . W_e
    grouped Wgrad  dW_e            = dY[o_e:o_{e+1}]^T . X[o_e:o_{e+1}]

Wgrad contracts over each expert's own tokens.  Its operands are grouped 1x128
along the tokens, and a group must not mix two experts: every expert's tokens
are quantized on their own, with a partial last group when m_e is not a
multiple of 128.

Token-padded layout of the Wgrad operands (a reading: the pages give no
grouped layout).  Expert e's m_e tokens occupy padded token columns
[p_e, p_e + m_e) with p_e = 128 * (floor(o_e / 128) + e).  The columns
[p_e + m_e, p_e + 128 * ceil(m_e / 128)) hold code 0.  Chunk j of the padded
axis (columns [128j, 128j + 128)) then belongs to at most one expert, and the
capacity 128 * (floor(M / 128) + E) bounds the padded axis.  Columns that
belong to no expert are not defined.
"""

import numpy as np

from .gemm import dgrad_ref, wgrad_ref
from .quant import quant_transpose

GROUP = 128


def padded_starts(offsets):
    """p_e = 128 * (floor(o_e / 128) + e) for e < E (int64 array)."""
    o = np.asarray(offsets, dtype=np.int64)[:-1]
    return GROUP * (o // GROUP + np.arange(len(o), dtype=np.int64))


def token_capacity(m_total, experts):
    """Length of the padded token axis: 128 * (floor(M / 128) + E)."""
    return GROUP * (int(m_total) // GROUP + int(experts))


def quant_transpose_grouped(x, offsets):
    """x float32 [M tokens, C channels], offsets [E+1] -> (q_t uint8 [C, cap],
    s_t float32 [C, cap/128], col_defined bool [cap], chunk_defined bool
    [cap/128]).  Each expert's token block is quantized with the 1x128 rule
    along the tokens (quant_transpose) and placed at its padded start;
    padding columns inside an expert's last chunk are code 0; undefined
    columns and chunks are left 0 and flagged False."""
    x = np.asarray(x, dtype=np.float32)
    offsets = np.asarray(offsets, dtype=np.int64)
    e_count = len(offsets) - 1
    cols = x.shape[1]
    cap = token_capacity(offsets[-1], e_count)
    q_t = np.zeros((cols, cap), dtype=np.uint8)
    s_t = np.zeros((cols, cap // GROUP), dtype=np.float32)
    col_def = np.zeros(cap, dtype=bool)
    chunk_def = np.zeros(cap // GROUP, dtype=bool)
    for e, p in enumerate(padded_starts(offsets)):
        lo, hi = int(offsets[e]), int(offsets[e + 1])
        m = hi - lo
        if m == 0:
            continue
        qe, se = quant_transpose(x[lo:hi])
        nc = (m + GROUP - 1) // GROUP
        q_t[:, p:p + m] = qe
        s_t[:, p // GROUP:p // GROUP + nc] = se
        col_def[p:p + nc * GROUP] = True
        chunk_def[p // GROUP:p // GROUP + nc] = True
    return q_t, s_t, col_def, chunk_def


def grouped_dgrad_ref(dyq, dys, wq_t, ws, offsets):
    """Per expert e: dX[o_e:o_{e+1}] = dY[o_e:o_{e+1}] . W_e.
    dyq [M, N], dys [M, N/128]; wq_t [K, E*N] = the transposed codes of the
    stacked weights [E*N, K] (expert e's W_e^T is columns [eN, (e+1)N)); ws
    [E*N/128, K/128] = the stacked block scales.  Returns (dX, S) float64."""
    offsets = np.asarray(offsets, dtype=np.int64)
    wq_t = np.asarray(wq_t)
    m_total = int(offsets[-1])
    n = dyq.shape[1]
    k = wq_t.shape[0]
    dx = np.zeros((m_total, k))
    s = np.zeros((m_total, k))
    for e in range(len(offsets) - 1):
        lo, hi = int(offsets[e]), int(offsets[e + 1])
        if hi == lo:
            continue
        w_e = wq_t[:, e * n:(e + 1) * n].T                   # forward layout [N, K]
        ws_e = ws[e * (n // GROUP):(e + 1) * (n // GROUP)]
        dx[lo:hi], s[lo:hi] = dgrad_ref(dyq[lo:hi], dys[lo:hi], w_e, ws_e)
    return dx, s


def grouped_wgrad_ref(dyq_t, dys_t, xq_t, xs_t, offsets):
    """Per expert e: dW_e = dY_e^T . X_e over the expert's own tokens, from the
    token-padded operands: dyq_t [N, cap], dys_t [N, cap/128], xq_t [K, cap],
    xs_t [K, cap/128].  Returns (dW [E, N, K], S [E, N, K]) float64; experts
    without tokens give zeros."""
    offsets = np.asarray(offsets, dtype=np.int64)
    e_count = len(offsets) - 1
    n, k = dyq_t.shape[0], xq_t.shape[0]
    dw = np.zeros((e_count, n, k))
    s = np.zeros((e_count, n, k))
    for e, p in enumerate(padded_starts(offsets)):
        m = int(offsets[e + 1] - offsets[e])
        if m == 0:
            continue
        nc = (m + GROUP - 1) // GROUP
        c0 = p // GROUP
        dw[e], s[e] = wgrad_ref(dyq_t[:, p:p + m], dys_t[:, c0:c0 + nc], xq_t[:, p:p + m], xs_t[:, c0:c0 + nc])
    return dw, s
