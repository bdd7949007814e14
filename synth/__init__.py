"""Seeded synthetic inputs shaped like the linear and MoE layers the pages
describe (activation outliers: the innerforce.co.kr excerpt of the DeepSeek-V3
report, paragraph on Figure 7 (a); token-correlated outliers in activation
gradients: "DeepSeek FP8 Training", last paragraph).

This module holds no arithmetic of the quantization method: it only draws
random tensors.  Both the oracle side and the GPU side of every test and of the
benchmark take their inputs from here.

All draws use ``numpy.random.Generator(PCG64(1000 + c))`` for configuration c,
in the order listed per configuration.  BF16 tensors are rounded from float32
to BF16 by round-to-nearest-even after the outliers are applied (torch's CPU
cast); weights stay float32.  Outlier counts are round(fraction * population)
distinct indices drawn without replacement.

Configurations (shapes are those of a 7168-wide model layer with a 2048-wide
projection and a 32-expert MoE layer):
  1 tiny Fprop     X [128,256] N(0,1), 33 entries x50;     W [128,256] N(0,0.02)
  2 linear Fprop   X [4096,7168] N(0,1), 143 channels x20; W [2048,7168] N(0,0.02)
  3 linear Dgrad   dY [4096,2048] Student-t(3), 41 rows x100; W as config 2
  4 linear Wgrad   X as config 2, dY as config 3
  5 MoE Fprop      W_e [32,2048,7168] N(0,0.02); X [16384,7168] N(0,1) sorted
                   by expert; counts: 4 dead experts, Zipf(1.1) over the other
                   28, no non-zero count a multiple of 128
  6 MoE backward   dY [16384,2048] Student-t(3), 164 token rows x100 (config 3's
                   recipe at config 5's token count); the expert offsets,
                   weights and X are config 5's
"""

import numpy as np
import torch

SEED_BASE = 1000


def rng_for(config):
    return np.random.Generator(np.random.PCG64(SEED_BASE + config))


def to_bf16(a):
    """float array -> torch.bfloat16 CPU tensor (float32 first, then RNE to BF16)."""
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(torch.bfloat16)


def _normal(rng, shape, std=1.0, out=None):
    """float32 N(0, std^2) draws (the float32 ziggurat of numpy)."""
    a = rng.standard_normal(shape, dtype=np.float32, out=out)
    if std != 1.0:
        a *= np.float32(std)
    return a


def tiny_fprop():
    """Config 1: returns (X bf16 [128,256], W float32 [128,256])."""
    rng = rng_for(1)
    x = _normal(rng, (128, 256))
    idx = rng.choice(x.size, size=round(0.001 * x.size), replace=False)
    x.reshape(-1)[idx] *= 50.0
    w = _normal(rng, (128, 256), 0.02).astype(np.float32)
    return to_bf16(x), torch.from_numpy(w)


def linear_x_w(m=4096, k=7168, n=2048):
    """Config 2: X bf16 [m,k] with 2% of channels x20, W float32 [n,k]."""
    rng = rng_for(2)
    x = _normal(rng, (m, k))
    ch = rng.choice(k, size=round(0.02 * k), replace=False)
    x[:, ch] *= 20.0
    w = _normal(rng, (n, k), 0.02).astype(np.float32)
    return to_bf16(x), torch.from_numpy(w)


def linear_dy(m=4096, n=2048):
    """Config 3: dY bf16 [m,n], Student-t(3) with 1% of rows (tokens) x100."""
    rng = rng_for(3)
    dy = rng.standard_t(3.0, size=(m, n))
    rows = rng.choice(m, size=round(0.01 * m), replace=False)
    dy[rows, :] *= 100.0
    return to_bf16(dy)


def moe_dy(tokens=16384, n=2048):
    """Config 6: dY bf16 [tokens, n] of the MoE layer, Student-t(3) with 1% of
    the token rows x100."""
    rng = rng_for(6)
    dy = rng.standard_t(3.0, size=(tokens, n))
    rows = rng.choice(tokens, size=round(0.01 * tokens), replace=False)
    dy[rows, :] *= 100.0
    return to_bf16(dy)


def moe_counts(rng, tokens=16384, experts=32, dead=4, zipf_s=1.1):
    """Per-expert token counts: `dead` experts get 0; the others get a
    multinomial draw with p proportional to rank^-s over a seeded rank
    permutation; then any non-zero count that is a multiple of 128 hands one
    token to the next live expert (repeated until none is left)."""
    dead_ids = rng.choice(experts, size=dead, replace=False)
    live = np.array([e for e in range(experts) if e not in set(dead_ids.tolist())])
    ranks = rng.permutation(len(live)) + 1
    p = ranks.astype(np.float64) ** (-zipf_s)
    p /= p.sum()
    counts = np.zeros(experts, dtype=np.int64)
    counts[live] = rng.multinomial(tokens, p)
    for _ in range(4 * experts):
        bad = [i for i, e in enumerate(live) if counts[e] > 0 and counts[e] % 128 == 0]
        if not bad:
            break
        i = bad[0]
        counts[live[i]] -= 1
        counts[live[(i + 1) % len(live)]] += 1
    assert counts.sum() == tokens
    assert (counts == 0).any()
    assert not any(c > 0 and c % 128 == 0 for c in counts)
    return counts


def moe_fprop(tokens=16384, experts=32, n=2048, k=7168, dead=4):
    """Config 5: returns (X bf16 [tokens,k] sorted by expert, W float32
    [experts,n,k], offsets int32 [experts+1])."""
    rng = rng_for(5)
    w = np.empty((experts, n, k), dtype=np.float32)
    for e in range(experts):
        _normal(rng, (n, k), 0.02, out=w[e])
    x = _normal(rng, (tokens, k))
    counts = moe_counts(rng, tokens, experts, dead)
    offsets = np.zeros(experts + 1, dtype=np.int32)
    offsets[1:] = np.cumsum(counts)
    return to_bf16(x), torch.from_numpy(w), torch.from_numpy(offsets)


def small_moe(tokens, experts, n, k, seed, dead=1):
    """A small seeded MoE case for parity tests: counts need not avoid
    multiples of 128; includes `dead` empty experts."""
    rng = np.random.Generator(np.random.PCG64(seed))
    w = _normal(rng, (experts, n, k), 0.02).astype(np.float32)
    x = _normal(rng, (tokens, k))
    cut = np.sort(rng.integers(0, tokens + 1, size=experts - 1))
    offsets = np.concatenate([[0], cut, [tokens]]).astype(np.int32)
    dead_ids = rng.choice(experts, size=dead, replace=False)
    counts = np.diff(offsets)
    for d in dead_ids:                   # fold a dead expert's rows into its neighbour
        if counts[d]:
            nb = (d + 1) % experts
            counts[nb] += counts[d]
            counts[d] = 0
    offsets = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    return to_bf16(x), torch.from_numpy(w), torch.from_numpy(offsets)


def general(rows, cols, seed, kind="normal", outlier_frac=0.0, outlier_mul=1.0):
    """A generic seeded float64 matrix for edge-shape tests."""
    rng = np.random.Generator(np.random.PCG64(seed))
    if kind == "t3":
        a = rng.standard_t(3.0, size=(rows, cols))
    else:
        a = rng.standard_normal((rows, cols))
    if outlier_frac and a.size:
        idx = rng.choice(a.size, size=max(1, round(outlier_frac * a.size)), replace=False)
        a.reshape(-1)[idx] *= outlier_mul
    return a
