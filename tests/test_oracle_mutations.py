"""Each test plants one plausible mistake in the oracle (on the CPU, through
monkeypatch) and checks that a pin catches it.  This shows the pins are tight
enough that a dropped term, a wrong index or a wrong rounding cannot pass."""
import numpy as np
import pytest

import oracle
import oracle.e4m3 as e4m3_mod
import oracle.gemm as gemm_mod
import oracle.quant as quant_mod
import oracle.sparse24 as sp_mod

import test_oracle_e4m3 as t_e4m3
import test_oracle_gemm as t_gemm
import test_oracle_quant as t_quant
import test_oracle_rowwise as t_row
import test_oracle_sparse24 as t_sp


_ROWWISE = gemm_mod._rowwise


def _fails(fn, *args):
    with pytest.raises(AssertionError):
        fn(*args)


def test_wrong_exponent_bias_is_caught(monkeypatch):
    bad = e4m3_mod._TABLE.copy()
    bad[8:0x7F] *= 2.0
    monkeypatch.setattr(e4m3_mod, "_TABLE", bad)
    _fails(t_e4m3.test_decode_all_256_codes_match_torch)


def test_ties_away_from_zero_is_caught(monkeypatch):
    def enc(v):
        v = np.asarray(v, np.float32)
        a = np.abs(v.astype(np.float64))
        lo = np.searchsorted(e4m3_mod._MID, a, side="right")   # ties go up
        code = np.minimum(lo, 0x7E).astype(np.uint8)
        return code | (np.signbit(v).astype(np.uint8) << 7)
    monkeypatch.setattr(oracle, "e4m3_encode", enc)
    _fails(t_e4m3.test_encode_midpoints_match_torch)


def test_inverted_scale_is_caught(monkeypatch):
    orig = quant_mod.fp8_quant_groupwise

    def quant(x, gr, gc):
        codes, s = orig(x, gr, gc)
        return codes, (np.float32(1.0) / s).astype(np.float32)
    monkeypatch.setattr(oracle, "fp8_quant_groupwise", quant)
    _fails(t_quant.test_power_of_two_roundtrip_is_exact)


def test_multiply_by_reciprocal_is_caught(monkeypatch):
    """v * (1/s) instead of v / s differs by an ulp now and then and can flip a tie."""
    def quant(x, gr, gc):
        x32 = np.asarray(x, np.float32)
        rows, cols = x32.shape
        amax = quant_mod._block_amax(x32, gr, gc)
        s = np.where(amax > 0, amax / np.float32(448), np.float32(1)).astype(np.float32)
        r = (np.float32(1) / s).astype(np.float32)
        q = (x32 * quant_mod._expand(r, gr, gc, rows, cols)).astype(np.float32)
        return oracle.e4m3_encode(q), s
    monkeypatch.setattr(oracle, "fp8_quant_groupwise", quant)
    _fails(t_quant.test_divide_not_reciprocal_on_a_tie)


def test_keeping_smallest_is_caught(monkeypatch):
    def prune(w):
        w = np.asarray(w)
        rows, k = w.shape
        mag = np.abs(sp_mod._values(w)).reshape(rows, k // 4, 4)
        order = np.argsort(mag, axis=-1, kind="stable")
        keep = np.zeros((rows, k // 4, 4), bool)
        np.put_along_axis(keep, order[..., :2], True, axis=-1)
        keep = keep.reshape(rows, k)
        return keep, np.where(keep, w, np.zeros((), w.dtype)).astype(w.dtype)
    monkeypatch.setattr(oracle, "prune24", prune)
    _fails(t_sp.test_prune_brute_force_all_groups)


def test_tie_to_higher_index_is_caught(monkeypatch):
    def prune(w):
        w = np.asarray(w)
        rows, k = w.shape
        mag = np.abs(sp_mod._values(w)).reshape(rows, k // 4, 4)[..., ::-1]
        order = 3 - np.argsort(-mag, axis=-1, kind="stable")
        keep = np.zeros((rows, k // 4, 4), bool)
        np.put_along_axis(keep, order[..., :2], True, axis=-1)
        keep = keep.reshape(rows, k)
        return keep, np.where(keep, w, np.zeros((), w.dtype)).astype(w.dtype)
    monkeypatch.setattr(oracle, "prune24", prune)
    _fails(t_sp.test_prune_brute_force_all_groups)


def test_swapped_nibble_order_is_caught(monkeypatch):
    """A layout mistake made consistently in compress and decompress survives
    every round trip; the hand-worked golden rows catch it."""
    orig_c = sp_mod.compress24

    def comp(w, keep):
        vals, meta = orig_c(w, keep)
        return vals, ((meta >> 4) | (meta << 4)).astype(np.uint8)
    monkeypatch.setattr(oracle, "prune_compress24", lambda w: comp(*oracle.prune24(w)[::-1]))
    _fails(t_sp.test_golden_hand_examples)


def test_dropped_last_k_block_is_caught(monkeypatch):
    orig = gemm_mod._scaled_kblock_sum

    def short(xd, sxe, wd, swe, absolute):
        return orig(xd[:, :-128], sxe[:, :-1], wd[:, :-128], swe[:, :-1], absolute) \
            if xd.shape[1] > 128 else 0 * orig(xd, sxe, wd, swe, absolute)
    monkeypatch.setattr(gemm_mod, "_scaled_kblock_sum", short)
    _fails(t_gemm.test_exact_rational_brute_force, 4, 2, 256, 1, 128)


def test_scale_block_index_off_is_caught(monkeypatch):
    """Using the next K block's W scale (a shifted index) is caught by the
    per-element-dequantisation route."""
    orig = gemm_mod.expand_scales

    def shifted(s, g, rows):
        e = orig(s, g, rows)
        return np.roll(e, 1, axis=1) if e.shape[0] > 200 else e
    monkeypatch.setattr(gemm_mod, "expand_scales", shifted)
    _fails(t_gemm.test_matches_per_element_dequantised_matmul, 1, 128)


def test_scale_granularity_ignored_is_caught(monkeypatch):
    """Treating granularity 128 as 1 (one scale row per matrix row) reads the
    wrong scales; the identity pin catches it."""
    orig = gemm_mod.expand_scales

    def no_repeat(s, g, rows):
        s = np.asarray(s, np.float32).astype(np.float64)
        out = np.zeros((rows, s.shape[1]))
        out[:min(rows, s.shape[0])] = s[:rows]
        return out
    monkeypatch.setattr(gemm_mod, "expand_scales", no_repeat)
    _fails(t_gemm.test_identity_dequantises_weight)


import test_oracle_int8 as t_int8  # noqa: E402


def test_int8_ties_away_from_zero_is_caught(monkeypatch):
    def quant(x, gr, gc):
        x32 = np.asarray(x, np.float32)
        rows, cols = x32.shape
        amax = quant_mod._block_amax(x32, gr, gc)
        s = np.where(amax > 0, amax / np.float32(127), np.float32(1)).astype(np.float32)
        q = (x32 / quant_mod._expand(s, gr, gc, rows, cols)).astype(np.float32)
        r = np.sign(q) * np.floor(np.abs(q) + 0.5)                       # ties away from zero
        return np.clip(r, -127, 127).astype(np.int8), s
    monkeypatch.setattr(oracle, "int8_quant_groupwise", quant)
    _fails(t_int8.test_int8_ties_round_to_even)


def test_int8_scale_by_128_is_caught(monkeypatch):
    def quant(x, gr, gc):
        x32 = np.asarray(x, np.float32)
        rows, cols = x32.shape
        amax = quant_mod._block_amax(x32, gr, gc)
        s = np.where(amax > 0, amax / np.float32(128), np.float32(1)).astype(np.float32)
        q = (x32 / quant_mod._expand(s, gr, gc, rows, cols)).astype(np.float32)
        return np.clip(np.rint(q), -127, 127).astype(np.int8), s
    monkeypatch.setattr(oracle, "int8_quant_groupwise", quant)
    _fails(t_int8.test_int8_power_of_two_roundtrip_is_exact)


def test_int8_shifted_kblock_scale_is_caught(monkeypatch):
    orig = gemm_mod.int8_gemm_groupwise

    def gemm(xq, sx, gm, wq, sw, gn, bound=False):
        return orig(xq, np.roll(np.asarray(sx), 1, axis=1), gm, wq, sw, gn, bound=bound)
    monkeypatch.setattr(oracle, "int8_gemm_groupwise", gemm)
    _fails(t_int8.test_int8_exact_rational_brute_force, 4, 2, 256, 1, 128)


def test_int8_dropped_sign_is_caught(monkeypatch):
    orig = gemm_mod.int8_gemm_groupwise

    def gemm(xq, sx, gm, wq, sw, gn, bound=False):
        return orig(np.abs(np.asarray(xq, np.int8).astype(np.int64)).astype(np.int8), sx, gm, wq, sw, gn, bound=bound)
    monkeypatch.setattr(oracle, "int8_gemm_groupwise", gemm)
    _fails(t_int8.test_int8_unit_scales_match_int64_matmul)


def test_rowwise_dropped_w_scale_is_caught(monkeypatch):
    def rowwise(xd, sx, wd, sw, bound):
        return _ROWWISE(xd, sx, wd, np.ones_like(np.asarray(sw, np.float32)), bound)
    monkeypatch.setattr(gemm_mod, "_rowwise", rowwise)
    _fails(t_row.test_rowwise_matches_exact_rationals, 3, 2, 128, False, False)


def test_rowwise_scale_of_wrong_row_is_caught(monkeypatch):
    def rowwise(xd, sx, wd, sw, bound):
        return _ROWWISE(xd, np.roll(np.broadcast_to(np.asarray(sx, np.float32), (xd.shape[0],)), 1), wd, sw, bound)
    monkeypatch.setattr(gemm_mod, "_rowwise", rowwise)
    _fails(t_row.test_rowwise_matches_exact_rationals, 3, 2, 128, False, False)


def test_rowwise_first_kblock_only_is_caught(monkeypatch):
    def rowwise(xd, sx, wd, sw, bound):
        return _ROWWISE(xd[:, :128], sx, wd[:, :128], sw, bound)
    monkeypatch.setattr(gemm_mod, "_rowwise", rowwise)
    _fails(t_row.test_rowwise_unit_scales_integer_codes_match_int64)


def test_rowwise_bound_without_abs_is_caught(monkeypatch):
    def rowwise(xd, sx, wd, sw, bound):
        y = _ROWWISE(xd, sx, wd, sw, False)
        return (y, y) if bound else y
    monkeypatch.setattr(gemm_mod, "_rowwise", rowwise)
    _fails(t_row.test_rowwise_bound_dominates_and_is_tight_for_nonnegative_codes)


def test_bias_on_rows_instead_of_columns_is_caught(monkeypatch):
    def add_bias(y, bound, bias):
        b = np.asarray(bias, np.float64)
        return y + np.resize(b, y.shape[0])[:, None], bound + np.abs(np.resize(b, y.shape[0]))[:, None]
    monkeypatch.setattr(oracle, "add_bias", add_bias)
    _fails(t_row.test_bias_adds_per_output_column_exactly_on_integers)


import test_oracle_w8a16 as t_w8  # noqa: E402


def test_w8a16_scale_of_wrong_kblock_is_caught(monkeypatch):
    orig = gemm_mod.w8a16_sparse24_gemm_groupwise

    def gemm(x_bits, wv, wmeta, sw, gn, codes="e4m3", bound=False):
        return orig(x_bits, wv, wmeta, np.roll(np.asarray(sw), 1, axis=1), gn, codes, bound)
    monkeypatch.setattr(oracle, "w8a16_sparse24_gemm_groupwise", gemm)
    _fails(t_w8.test_w8a16_matches_exact_rationals, False, 128)


def test_w8a16_int8_read_unsigned_is_caught(monkeypatch):
    orig = gemm_mod.w8a16_sparse24_gemm_groupwise

    def gemm(x_bits, wv, wmeta, sw, gn, codes="e4m3", bound=False):
        if codes == "int8":
            wq = oracle.decompress24(np.asarray(wv).view(np.uint8), wmeta).astype(np.float64)
            y = oracle.bf16_decode(x_bits) @ wq.T * np.float64(np.asarray(sw).reshape(-1)[0])
            return (y, np.abs(y)) if bound else y
        return orig(x_bits, wv, wmeta, sw, gn, codes, bound)
    monkeypatch.setattr(oracle, "w8a16_sparse24_gemm_groupwise", gemm)
    _fails(t_w8.test_w8a16_integer_activations_int8_codes_unit_scales)


def test_w4a16_nibbles_swapped_is_caught(monkeypatch):
    def w4(x_bits, wv4, wmeta, sw, bound=False):
        b = np.asarray(wv4, np.uint8)
        swapped = ((b >> 4) | (b << 4)).astype(np.uint8)
        codes = oracle.int4_decode(swapped).astype(np.int8)
        return oracle.w8a16_sparse24_gemm_groupwise(x_bits, codes, wmeta, sw, 1, "int8", bound=bound)
    monkeypatch.setattr(oracle, "w4a16_sparse24_gemm_groupwise", w4)
    _fails(t_w8.test_w4a16_matches_exact_rationals)


def test_nan_ranked_as_zero_is_caught(monkeypatch):
    """A pruner that ranks |w| with NaN treated as the smallest magnitude (what
    an fmax-style comparison does) drops NaN weights."""
    def prune(w):
        w = np.asarray(w)
        rows, k = w.shape
        mag = np.nan_to_num(np.abs(sp_mod._values(w)), nan=-1.0).reshape(rows, k // 4, 4)
        order = np.argsort(-mag, axis=-1, kind="stable")
        keep = np.zeros((rows, k // 4, 4), bool)
        np.put_along_axis(keep, order[..., :2], True, axis=-1)
        keep = keep.reshape(rows, k)
        return keep, np.where(keep, w, np.zeros((), w.dtype)).astype(w.dtype)
    monkeypatch.setattr(oracle, "prune24", prune)
    _fails(t_sp.test_prune_brute_force_nonfinite)


def test_amax_that_skips_nan_is_caught(monkeypatch):
    """np.nanmax-style block maxima hide a NaN: the block gets a finite scale."""
    orig = quant_mod._block_amax

    def amax(x32, gr, gc):
        return orig(np.nan_to_num(x32, nan=0.0), gr, gc)
    monkeypatch.setattr(quant_mod, "_block_amax", amax)
    _fails(t_quant.test_nonfinite_blocks_follow_ieee_through_the_formulas)
