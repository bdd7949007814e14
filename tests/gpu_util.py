"""Shared helpers of the GPU parity tests: move seeded inputs to the GPU, run the
oracle on the same inputs, and compare element by element."""

import json
import math
import os

import numpy as np
import torch

DEV = "cuda:0"
REL_TOL = 1e-5          # |y - Y_ref| <= 1e-5 * sum_k |a_k b_k|
ERR_LOG = os.environ.get("FP8Q_ERR_LOG")  # if set: every GEMM check appends its error statistics (JSON lines)


def gpu(t):
    return t.to(DEV)


def f32(t):
    """BF16/FP32 torch tensor -> float32 numpy (exact widening)."""
    return t.detach().float().cpu().numpy()


def np_u8(t):
    return t.detach().cpu().numpy()


def assert_bytes_equal(got, want, what):
    got = np.asarray(got)
    want = np.asarray(want)
    assert got.shape == want.shape, (what, got.shape, want.shape)
    bad = np.nonzero(got.reshape(-1) != want.reshape(-1))[0]
    assert bad.size == 0, f"{what}: {bad.size} mismatches, first at flat {bad[:5].tolist()}: " \
                          f"got {got.reshape(-1)[bad[:5]].tolist()} want {want.reshape(-1)[bad[:5]].tolist()}"


def assert_scales_equal(got, want, what):
    got = np.asarray(got, np.float32)
    want = np.asarray(want, np.float32)
    assert_bytes_equal(got.view(np.uint32), want.view(np.uint32), what)


def bf16_ulp(v):
    a = np.abs(np.asarray(v, np.float64))
    e = np.floor(np.log2(np.where(a > 0, a, 1.0)))
    e = np.where(a > 0, np.maximum(e, -126), -126)
    return np.exp2(e - 7)


def check_gemm(y, y_ref, s_ref, out_bf16, what, exact=True, nk=None, strict=False):
    """Elementwise bar, S = sum_k |a_k b_k| of the exact contraction.

    exact=True (the *_exact entry points): FP32 output |y - Y_ref| <= 1e-5 S;
    BF16 output |y - Y_ref| <= ulp_bf16(Y_ref) + 1e-5 S.

    exact=False (the FP8 matrix-instruction entry points): gfx950's FP8 MFMA
    keeps 14 bits below the largest of each group of 8 products and truncates
    the rest, so each group may lose < 7 * 2^-13 of its largest product:
    |y - Y_ref| <= 2^-10 S + (nk + 17) 2^-24 S (+ ulp_bf16 for BF16 output),
    and for FP32 output the mean of |y - Y_ref| / S must stay below 5e-5.

    strict=True (FP8 entry points on the configurations' full-size BF16
    products, where it holds): the exact bar as well, no element outside
    ulp_bf16(Y_ref) + 1e-5 S."""
    y = np.asarray(y, np.float64)
    err = np.abs(y - y_ref)
    s = np.maximum(s_ref, 1e-300)
    if exact:
        bound = REL_TOL * s_ref
    else:
        bound = (2.0 ** -10 + ((nk or 0) + 17) * 2.0 ** -24) * s_ref
    if out_bf16:
        bound = bound + bf16_ulp(y_ref)
    over = err > bound
    stats = {
        "what": what + (" exact" if exact else " fp8"),
        "n": int(y.size),
        "max_err_over_S": float((err / s).max()) if y.size else 0.0,
        "mean_err_over_S": float((err / s).mean()) if y.size else 0.0,
        "n_over": int(over.sum()),
        "n_over_1e-5_S": int((err > REL_TOL * s_ref + (bf16_ulp(y_ref) if out_bf16 else 0.0)).sum()),
    }
    if out_bf16:
        rne = torch.from_numpy(y_ref.astype(np.float32)).to(torch.bfloat16).double().numpy()
        stats["n_not_rne_of_ref"] = int((y != rne).sum())
    print("GEMM", stats, flush=True)
    if ERR_LOG:
        with open(ERR_LOG, "a") as f:
            f.write(json.dumps(stats) + "\n")
    if over.any():
        idx = np.argwhere(over)[:5]
        detail = [(tuple(int(v) for v in i), float(y[tuple(i)]), float(y_ref[tuple(i)]), float(s_ref[tuple(i)]))
                  for i in idx]
        raise AssertionError(f"{what}: {int(over.sum())} of {y.size} outside tolerance; first: {detail}")
    if not exact and not out_bf16 and y.size:
        assert stats["mean_err_over_S"] <= 5e-5, stats
    if strict:
        assert stats["n_over_1e-5_S"] == 0, stats
    return stats


def sample_rows(n, k, seed, must=()):
    rng = np.random.Generator(np.random.PCG64(seed))
    rows = set(int(r) for r in must if 0 <= r < n)
    rows.update(int(r) for r in rng.choice(n, size=min(k, n), replace=False))
    return np.array(sorted(rows), dtype=np.int64)


def log(msg):
    print(msg, flush=True)


def case_name(*parts):
    return "-".join(str(p) for p in parts)


def isclose(a, b):
    return math.isclose(a, b, rel_tol=0, abs_tol=0)
