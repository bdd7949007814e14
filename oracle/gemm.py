"""GEMM references of the oracle (test infrastructure only).

What the method computes ("DeepSeek FP8 Training", the Fprop pipeline list and
the weight- and input-gradient lists; the innerforce.co.kr excerpt, paragraph
after Figure 7 (a): dequantization is folded into the FP32 accumulation):

    Fprop   Y [M,N]  = X  [M,K] . W^T          X: 1x128 groups, W: 128x128 blocks
    Dgrad   dX[M,K]  = dY [M,N] . W             dY: 1x128 groups
    Wgrad   dW[N,K]  = dY^T . X  over T tokens  both operands grouped 1x128
                                                along the tokens
    Grouped Y[o_e:o_e+1] = X[o_e:o_e+1] . W_e^T per expert e

with every operand replaced by its dequantized value dec(q) * s(group).  The
result is the plain contraction of the dequantized operands; promoting FP32
partials every 128 K (the "unified E4M3 format" page, section "Enhanced
Numerical Stability") is how a kernel gets close to it, so it is not part of
this definition.  Each dequantized value has at most 28 significant bits, so
float64 holds it exactly; the sums are float64 matmuls (host BLAS).

Each reference also returns S = sum_k |a_mk * b_nk| (float64), the scale of
the rounding error of any summation order, used to normalise tolerances.

``exact_outputs`` gives chosen outputs as exact rationals: dec(code) * 2^9 is
an integer of magnitude <= 229376, so a 128-long chunk dot product is an exact
int64, and the chunk sums are combined with the FP32 scales in
``fractions.Fraction``.
"""

from fractions import Fraction

import numpy as np

from .e4m3 import decode

GROUP = 128


def _deq_rows(q, s):
    """q [R, C] codes grouped 1x128 along C, s [R, ceil(C/128)] -> float64."""
    q = np.asarray(q)
    cols = q.shape[1]
    idx = np.arange(cols) // GROUP
    return decode(q) * np.asarray(s, dtype=np.float64)[:, idx]


def _deq_blocks(q, s):
    """q [R, C] codes in 128x128 blocks, s [ceil(R/128), ceil(C/128)] -> float64."""
    q = np.asarray(q)
    ri = np.arange(q.shape[0]) // GROUP
    ci = np.arange(q.shape[1]) // GROUP
    return decode(q) * np.asarray(s, dtype=np.float64)[ri][:, ci]


def fprop_ref(xq, xs, wq, ws):
    """Y = X W^T.  xq [M,K], xs [M,K/128]; wq [N,K], ws [N/128,K/128]."""
    a = _deq_rows(xq, xs)
    b = _deq_blocks(wq, ws)
    return a @ b.T, np.abs(a) @ np.abs(b).T


def dgrad_ref(dyq, dys, wq, ws):
    """dX = dY W.  dyq [M,N], dys [M,N/128]; wq [N,K], ws [N/128,K/128]
    (the weight codes in their forward layout)."""
    a = _deq_rows(dyq, dys)
    w = _deq_blocks(wq, ws)
    return a @ w, np.abs(a) @ np.abs(w)


def wgrad_ref(dyq_t, dys_t, xq_t, xs_t):
    """dW = dY^T X over the tokens.  dyq_t [N,T], dys_t [N,T/128];
    xq_t [K,T], xs_t [K,T/128] (token-grouped, transposed codes)."""
    dy_t = _deq_rows(dyq_t, dys_t)        # [N, T] = dY^T
    x_t = _deq_rows(xq_t, xs_t)           # [K, T] = X^T
    return dy_t @ x_t.T, np.abs(dy_t) @ np.abs(x_t).T


def grouped_ref(xq, xs, wq, ws, offsets):
    """Per expert e: Y[o_e:o_{e+1}] = X[o_e:o_{e+1}] W_e^T.
    wq [E,N,K], ws [E,N/128,K/128], offsets [E+1] non-decreasing."""
    offsets = np.asarray(offsets, dtype=np.int64)
    m_total = int(offsets[-1])
    n = wq.shape[1]
    y = np.zeros((m_total, n))
    s = np.zeros((m_total, n))
    for e in range(len(offsets) - 1):
        lo, hi = int(offsets[e]), int(offsets[e + 1])
        if hi > lo:
            y[lo:hi], s[lo:hi] = fprop_ref(xq[lo:hi], xs[lo:hi], wq[e], ws[e])
    return y, s


def exact_outputs(qa, sa, qb, sb, pairs):
    """Exact values of C[m,n] = sum_k dec(qa[m,k]) sa[m,k/128] dec(qb[n,k]) sb[n,k/128]
    for the (m, n) in ``pairs``.  qa [M,K], qb [N,K] are codes with the
    contraction axis last; sa [M,K/128] and sb [N,K/128] give the FP32 scale
    of every (row, chunk).  Returns a list of Fractions."""
    qa = np.asarray(qa)
    qb = np.asarray(qb)
    k = qa.shape[1]
    nchunk = (k + GROUP - 1) // GROUP
    out = []
    for m, n in pairs:
        ia = (decode(qa[m]) * 512.0).astype(np.int64)
        ib = (decode(qb[n]) * 512.0).astype(np.int64)
        total = Fraction(0)
        for kb in range(nchunk):
            lo, hi = kb * GROUP, min(k, (kb + 1) * GROUP)
            dot = int(np.dot(ia[lo:hi], ib[lo:hi]))
            if dot:
                total += Fraction(dot) * Fraction(float(sa[m, kb])) * Fraction(float(sb[n, kb]))
        out.append(total / (1 << 18))
    return out
