"""Seeded matrices made of 128x128 tiles, each tile filled with one special
pattern, so that every grouping (1x128 rows, 128x128 blocks, 128x1 columns)
meets the same cases: the group max-abs mapped to 448 (the innerforce.co.kr
excerpt of the DeepSeek-V3 report, paragraph on Figure 7 (a)) at the edges of
FP32 and E4M3 range, where underflow and overflow happen ("DeepSeek FP8
Training", list of challenges)."""

import numpy as np

FLT_MAX = np.float32(3.4028235e38)
BF16_MAX = np.float32(3.3895314e38)

# E4M3FN grid (finite magnitudes), for values at rounding midpoints
_GRID = np.array(sorted({(8 + f) * 2.0 ** (e - 10) if e else f * 2.0 ** -9
                         for e in range(16) for f in range(8) if not (e == 15 and f == 7)}), np.float64)


def bf16_round(a):
    """FP32 -> nearest BF16 value (ties to even), as FP32."""
    u = np.asarray(a, np.float32).view(np.uint32).astype(np.uint64)
    u = ((u + 0x7FFF + ((u >> 16) & 1)) >> 16) << 16
    return u.astype(np.uint32).view(np.float32)


def _saturating_amax(rng, n, for_bf16):
    """Max-abs values whose FP32 product with fl32(448/amax) exceeds 448, so
    that the group maximum only lands on 448 through saturation (BF16 values
    when the matrix is meant for BF16 input)."""
    out = []
    while len(out) < n:
        a = np.float32(rng.uniform(1e-3, 1e3))
        if for_bf16:
            a = np.float32(bf16_round(a))
        inv = np.float32(np.float32(448.0) / a)
        if np.float32(a * inv) > np.float32(448.0):
            out.append(a)
    return np.array(out, np.float32)


PATTERNS = ["zero", "neg_zero", "mixed_zero", "denormal", "near_max", "one_outlier", "saturating",
            "wide_pow2", "big", "small", "constant", "midpoints", "neg_underflow"]


def _tile(kind, rng, for_bf16):
    t = np.zeros((128, 128), np.float32)
    top = BF16_MAX if for_bf16 else FLT_MAX
    if kind == "neg_zero":
        t[:] = -0.0
    elif kind == "mixed_zero":
        t[:] = np.where(rng.random((128, 128)) < 0.5, np.float32(-0.0), np.float32(0.0))
    elif kind == "denormal":
        # every max-abs below the 2^-100 floor: all codes +-0
        t[:] = rng.choice(np.array([1e-45, -1e-45, 3e-42, -2e-40, 1e-39, 0.0], np.float32), size=(128, 128))
    elif kind == "near_max":
        t[:] = (rng.uniform(0.25, 1.0, (128, 128)) * top).astype(np.float32) * rng.choice([-1, 1], (128, 128))
        t[0, 0] = top
    elif kind == "one_outlier":
        # one large value per row and column group; the rest far below it (subnormal codes, underflow to +-0)
        t[:] = (rng.standard_normal((128, 128)) * 1e-3).astype(np.float32)
        t[np.arange(128), rng.permutation(128)] = np.float32(1e4) * rng.choice([-1, 1], 128)
    elif kind == "saturating":
        # every row and every column holds one maximum whose scaled value rounds above 448
        a = _saturating_amax(rng, 128, for_bf16)
        t[:] = (rng.uniform(-1, 1, (128, 128)) * 1e-3).astype(np.float32)
        # row i's maximum sits in column perm[i]: every column group holds one too
        t[np.arange(128), rng.permutation(128)] = a * rng.choice([-1, 1], 128)
    elif kind == "wide_pow2":
        t[:] = np.exp2(rng.integers(-60, 61, (128, 128))).astype(np.float32) * rng.choice([-1, 1], (128, 128))
    elif kind == "big":
        t[:] = (rng.standard_normal((128, 128)) * 2.0 ** 60).astype(np.float32)
    elif kind == "small":
        t[:] = (rng.standard_normal((128, 128)) * 2.0 ** -60).astype(np.float32)
    elif kind == "constant":
        t[:] = np.float32(3.0)
    elif kind == "midpoints":
        # a 448 in every row and column (scale exactly 1) and values at midpoints of the E4M3 grid:
        # round-to-nearest-even decides every one of them
        mids = ((_GRID[:-1] + _GRID[1:]) / 2).astype(np.float32)
        t[:] = rng.choice(mids, (128, 128)) * rng.choice([-1, 1], (128, 128)).astype(np.float32)
        t[np.arange(128), rng.permutation(128)] = np.float32(448.0)
    elif kind == "neg_underflow":
        # negative values that round to zero keep their sign (code 0x80)
        t[:] = -np.float32(1e-9) * rng.random((128, 128)).astype(np.float32)
        t[np.arange(128), rng.permutation(128)] = np.float32(1.0)
    elif kind != "zero":
        raise ValueError(kind)
    return t


def special_matrix(rows, cols, seed, for_bf16=False):
    """[rows, cols] FP32 matrix of 128x128 special tiles, patterns cycling over
    the tiles (partial tiles at the edges keep their top-left part)."""
    rng = np.random.Generator(np.random.PCG64(seed))
    tr, tc = (rows + 127) // 128, (cols + 127) // 128
    out = np.zeros((tr * 128, tc * 128), np.float32)
    for i in range(tr):
        for j in range(tc):
            kind = PATTERNS[(i * tc + j) % len(PATTERNS)]
            out[128 * i:128 * i + 128, 128 * j:128 * j + 128] = _tile(kind, rng, for_bf16)
    return out[:rows, :cols].copy()
