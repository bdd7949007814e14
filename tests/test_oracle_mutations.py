"""Planted mistakes in the oracle (on the CPU only): each plausible error must
make at least one pin fail, which shows the pins are not vacuous."""

import numpy as np
import pytest

import oracle
from oracle import e4m3, gemm, quant

import test_oracle_codec as codec_pins
import test_oracle_gemm as gemm_pins
import test_oracle_quant as quant_pins


def _fails(fn, *args):
    with pytest.raises(AssertionError):
        fn(*args)


def test_wrong_exponent_bias_is_caught(monkeypatch):
    real = e4m3.decode
    monkeypatch.setattr(e4m3, "decode", lambda c: real(c) * 2.0)
    _fails(codec_pins.test_golden_decode_values)


def test_round_half_away_is_caught(monkeypatch):
    real_rint = np.rint

    class _NP:
        def __getattr__(self, k):
            return getattr(np, k)

        @staticmethod
        def rint(v):
            return np.floor(np.asarray(v) + 0.5)

    monkeypatch.setattr(e4m3, "np", _NP())
    _fails(codec_pins.test_encode_matches_brute_force)
    assert real_rint is np.rint


def test_divide_by_scale_convention_is_caught(monkeypatch):
    """Quantizing with x / s instead of x * fl32(448/amax') is a different,
    equally plausible reading; the pinned convention must tell them apart."""
    def by_division(x):
        x = np.asarray(x, np.float32)
        q, s = np.zeros(x.shape, np.uint8), np.zeros((x.shape[0], (x.shape[1] + 127) // 128), np.float32)
        for j in range(s.shape[1]):
            blk = x[:, 128 * j:128 * (j + 1)]
            sj, _ = quant.group_scale(np.abs(blk).max(axis=1))
            q[:, 128 * j:128 * (j + 1)] = e4m3.encode(np.divide(blk, sj[:, None], dtype=np.float32))
            s[:, j] = sj
        return q, s

    x = quant_pins._bf16_values(quant_pins.synth.general(64, 1024, seed=99, kind="t3"))
    q1, _ = quant.quant_act_1x128(x)
    q2, _ = by_division(x)
    assert not np.array_equal(q1, q2), "the two conventions should differ somewhere"
    monkeypatch.setattr(quant, "quant_act_1x128", by_division)
    _fails(quant_pins.test_act_matches_exact_rederivation)


def test_transposed_block_scale_is_caught(monkeypatch):
    def deq_blocks_t(q, s):
        s = np.asarray(s, np.float64)
        ri = np.arange(q.shape[0]) // 128
        ci = np.arange(q.shape[1]) // 128
        # row-block and column-block indices swapped (wrapped to stay in range)
        return e4m3.decode(q) * s[(ci % s.shape[0])[None, :], (ri % s.shape[1])[:, None]]
    monkeypatch.setattr(gemm, "_deq_blocks", deq_blocks_t)
    _fails(gemm_pins.check_fprop_pow2)


def test_dgrad_with_transposed_weight_is_caught(monkeypatch):
    def wrong(dyq, dys, wq, ws):
        a = gemm._deq_rows(dyq, dys)
        w = gemm._deq_blocks(wq, ws)
        k = w.shape[1]
        wt = np.zeros_like(w)
        mn = min(w.shape)
        wt[:mn, :mn] = w[:mn, :mn].T
        return a @ wt[:, :k], np.abs(a) @ np.abs(w)
    monkeypatch.setattr(oracle, "dgrad_ref", wrong)
    _fails(gemm_pins.check_dgrad_pow2)


def test_wgrad_grouping_on_wrong_axis_is_caught(monkeypatch):
    def wrong_transpose(x):
        q, s = quant.quant_act_1x128(np.asarray(x, np.float32))   # groups along channels
        g = (x.shape[0] + 127) // 128
        s_t = np.repeat(s[:1, :1], x.shape[1] * g).reshape(x.shape[1], g)
        return np.ascontiguousarray(q.T), s_t
    monkeypatch.setattr(oracle, "quant_transpose", wrong_transpose)
    _fails(gemm_pins.check_wgrad_pow2)


def test_dropped_chunk_is_caught(monkeypatch):
    real = gemm._deq_rows

    def drop_last_chunk(q, s):
        a = real(q, s)
        a[:, -128:] = 0.0
        return a
    monkeypatch.setattr(gemm, "_deq_rows", drop_last_chunk)
    _fails(gemm_pins.check_tiny_config_exact)


def test_sign_error_in_grouped_is_caught(monkeypatch):
    real = oracle.grouped_ref

    def flipped(*a):
        y, s = real(*a)
        return -y, s
    monkeypatch.setattr(oracle, "grouped_ref", flipped)
    _fails(gemm_pins.check_grouped_pow2)


# ----------------------------------------------------- grouped (MoE) backward
import test_oracle_grouped as grouped_pins  # noqa: E402
from oracle import grouped  # noqa: E402


def test_overlapping_padded_layout_is_caught(monkeypatch):
    """Padded starts without the per-expert extra chunk overlap."""
    monkeypatch.setattr(grouped, "padded_starts",
                        lambda off: 128 * (np.asarray(off, np.int64)[:-1] // 128))
    monkeypatch.setattr(oracle, "padded_starts", grouped.padded_starts)
    _fails(grouped_pins.test_padded_layout_never_overlaps)


def test_groups_straddling_experts_are_caught(monkeypatch):
    """Quantizing the concatenated tokens in global 128-token groups (a group
    may mix two experts) instead of each expert on its own."""
    def straddling(x, offsets):
        q_all, s_all = quant.quant_transpose(x)
        off = np.asarray(offsets, np.int64)
        cap = grouped.token_capacity(off[-1], len(off) - 1)
        q_t = np.zeros((x.shape[1], cap), np.uint8)
        s_t = np.zeros((x.shape[1], cap // 128), np.float32)
        for e, p in enumerate(grouped.padded_starts(off)):
            lo, hi = int(off[e]), int(off[e + 1])
            q_t[:, p:p + hi - lo] = q_all[:, lo:hi]
            for j in range(-(-(hi - lo) // 128)):
                s_t[:, p // 128 + j] = s_all[:, min((lo + 128 * j) // 128, s_all.shape[1] - 1)]
        return q_t, s_t, np.ones(cap, bool), np.ones(cap // 128, bool)

    monkeypatch.setattr(oracle, "quant_transpose_grouped", straddling)
    _fails(grouped_pins.test_grouped_transpose_matches_exact_rederivation)


def test_dgrad_with_first_expert_scales_is_caught(monkeypatch):
    """Using expert 0's block scales for every expert."""
    real = oracle.grouped_dgrad_ref

    def wrong(dyq, dys, wq_t, ws, offsets):
        n = dyq.shape[1]
        return real(dyq, dys, wq_t, np.tile(ws[:n // 128], (len(offsets) - 1, 1)), offsets)

    monkeypatch.setattr(oracle, "grouped_dgrad_ref", wrong)
    _fails(grouped_pins.test_grouped_dgrad_closed_form)


def test_wgrad_chunk_offset_error_is_caught(monkeypatch):
    """Reading an expert's token scales one chunk late."""
    real = oracle.grouped_wgrad_ref

    def shifted(dyq_t, dys_t, xq_t, xs_t, offsets):
        return real(dyq_t, np.roll(dys_t, 1, axis=1), xq_t, xs_t, offsets)

    monkeypatch.setattr(oracle, "grouped_wgrad_ref", shifted)
    _fails(grouped_pins.test_grouped_wgrad_closed_form)


# ------------------------------------------------------------ microscaling
import test_oracle_mx as mx_pins  # noqa: E402
from oracle import mx  # noqa: E402


def test_mx_exponent_off_by_one_is_caught(monkeypatch):
    """E4M3's largest power of two taken as 2^7 instead of 2^8."""
    real = mx.e8m0_of_amax
    monkeypatch.setattr(mx, "e8m0_of_amax", lambda a: np.minimum(real(a).astype(int) + 1, 254).astype(np.uint8))
    _fails(mx_pins.test_block_maximum_lands_in_the_top_binade)


def test_mx_truncating_conversion_is_caught(monkeypatch):
    real = e4m3.encode
    monkeypatch.setattr(mx, "encode", lambda y: real(np.trunc(np.asarray(y, np.float64) * 4) / 4))
    _fails(mx_pins.test_codes_match_brute_force, 0)
