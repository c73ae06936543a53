"""Each test plants one plausible mistake in the oracle (on the CPU, through
monkeypatch) and checks that at least one pin then fails. This shows the pins
are sensitive to dropped terms, wrong signs, wrong indices and transposed
operands, not only that the oracle passes them."""

import numpy as np
import pytest

from oracle import qblk_oracle as o
from tests import test_oracle_invariants as inv
from tests import test_oracle_pins as pins


def _round_half_even(v):
    return np.round(np.asarray(v, np.float64))


def test_mutant_round_half_even_is_caught(monkeypatch):
    monkeypatch.setattr(o, "round_half_away", _round_half_even)
    with pytest.raises(AssertionError):
        pins.test_round_half_away_matches_decimal()


def test_mutant_q4_0_divides_by_8_is_caught(monkeypatch):
    monkeypatch.setattr(o, "quantize_q4_0", lambda w: o.quantize_symmetric(w, 8))
    with pytest.raises(AssertionError):
        pins.test_q4_0_example_symmetric_rule()


def test_mutant_swapped_nibbles_is_caught(monkeypatch):
    def swapped(codes):
        c = np.asarray(codes, np.int64)
        return (c[..., 1::2] | (c[..., 0::2] << 4)).astype(np.uint8)
    monkeypatch.setattr(o, "_nibble_pairs", swapped)
    with pytest.raises(AssertionError):
        pins.test_q4_0_pack_matches_page_scalar_kernel()


def test_mutant_missing_offset_8_is_caught(monkeypatch):
    orig = o.pack_q4_0

    def no_offset(q, d):
        # stores the two's-complement low nibble instead of q + 8
        return orig((np.asarray(q) & 15) - 8, d)
    monkeypatch.setattr(o, "pack_q4_0", no_offset)
    with pytest.raises(AssertionError):
        pins.test_q4_0_pack_matches_page_scalar_kernel()


def test_mutant_dropped_q4_k_min_term_is_caught(monkeypatch):
    def no_min(enc, aq, da, sa):
        scale, _ = o.q4_k_sub_scales(enc)
        S = o.block_sums(enc["q"], aq).astype(np.float64)
        y = np.einsum("mnb,nb,mb->mn", S, scale, np.asarray(da, np.float64))
        return y.astype(np.float32), y
    monkeypatch.setattr(o, "product_q4_k", no_min)
    with pytest.raises(AssertionError):
        inv.test_product_equals_dequantized_dot(o.TYPE_Q4_K)


def test_mutant_wrong_dmin_sign_is_caught(monkeypatch):
    orig = o.quantize_q4_k

    def pos_dmin(w):
        enc = orig(w)
        enc["dmin_bits"] = enc["dmin_bits"] & 0x7FFF
        return enc
    monkeypatch.setattr(o, "quantize_q4_k", pos_dmin)
    with pytest.raises(AssertionError):
        inv.test_q4_k_round_trip_bound_and_ranges()


def test_mutant_transposed_block_sums_is_caught(monkeypatch):
    def transposed(wq, aq):
        wq = np.asarray(wq, np.int64)
        aq = np.asarray(aq, np.int64)
        N, K = wq.shape
        M = aq.shape[0]
        nb = K // 32
        r = np.einsum("mbi,nbi->nmb", aq.reshape(M, nb, 32), wq.reshape(N, nb, 32))
        return r.reshape(M, N, nb)
    monkeypatch.setattr(o, "block_sums", transposed)
    with pytest.raises(AssertionError):
        inv.test_block_sums_brute_force(o.TYPE_Q8_0, 3, 256, 5)


def test_mutant_block_index_off_by_one_is_caught(monkeypatch):
    orig = o.block_sums

    def shifted(wq, aq):
        return np.roll(orig(wq, aq), 1, axis=-1)
    monkeypatch.setattr(o, "block_sums", shifted)
    with pytest.raises(AssertionError):
        inv.test_product_equals_dequantized_dot(o.TYPE_Q4_0)


def test_mutant_sub_scale_index_is_caught(monkeypatch):
    orig = o.q4_k_sub_scales

    def rolled(enc):
        s, m = orig(enc)
        return np.roll(s, 1, axis=-1), m
    monkeypatch.setattr(o, "q4_k_sub_scales", rolled)
    with pytest.raises(AssertionError):
        inv.test_q4_k_hand_built_block_dequant()


def test_mutant_fp16_nearest_instead_of_ceiling_is_caught(monkeypatch):
    def nearest(v, c):
        h = (np.asarray(v, np.float64) / c).astype(np.float16)
        return h.view(np.uint16).astype(np.int64)
    monkeypatch.setattr(o, "f16_ceil_div", nearest)
    with pytest.raises(AssertionError):
        pins.test_f16_ceil_div_brute_force()


def test_mutant_activation_sum_of_abs_is_caught(monkeypatch):
    orig = o.quantize_act

    def abs_sum(x):
        q, d, s = orig(x)
        M, K = q.shape
        return q, d, np.abs(q).reshape(M, K // 32, 32).sum(-1)
    monkeypatch.setattr(o, "quantize_act", abs_sum)
    with pytest.raises(AssertionError):
        inv.test_block_sums_brute_force(o.TYPE_Q4_K, 2, 512, 2)


def test_mutant_group8_order_is_caught(monkeypatch):
    monkeypatch.setattr(o, "GROUP8_ORDER", np.array([0, 1, 2, 3, 4, 5, 6, 7]))
    with pytest.raises(AssertionError):
        inv.test_activation_buffer_layout()


def test_mutant_q4_0_f16_codes_against_fp32_scale_is_caught(monkeypatch):
    """Codes taken against the unrounded fp32 scale instead of the stored
    fp16 one: some element is then not at its nearest multiple of d16."""
    def mutant(w):
        q, d32 = o.quantize_symmetric(w, 7)
        return q, o.fp16_round(d32)
    monkeypatch.setattr(o, "quantize_q4_0_f16", mutant)
    with pytest.raises(AssertionError):
        inv.test_q4_0_f16_round_trip_bound_and_ranges()


def test_mutant_q4_0_f16_truncated_scale_is_caught(monkeypatch):
    """fp16 scale by truncation instead of rounding to nearest."""
    def trunc16(x):
        x = np.asarray(x, np.float32)
        h = x.astype(np.float16)
        over = np.abs(h.astype(np.float32)) > np.abs(x)
        step = np.nextafter(h, np.float16(0))
        return np.where(over, step, h).astype(np.float32)
    monkeypatch.setattr(o, "fp16_round", trunc16)
    with pytest.raises(AssertionError):
        pins.test_q4_0_f16_scale_is_nearest_half_of_amax_over_7()


def test_mutant_float_product_without_offset_8_is_caught(monkeypatch):
    """The float product decoding Q4_0 nibbles without the offset of 8."""
    def no_offset(wtype, enc, x):
        deq = (np.asarray(enc["q"], np.float64) + 8) * np.repeat(np.asarray(enc["d"], np.float64), 32, axis=1)
        y = np.asarray(x, np.float64) @ deq.T
        return y.astype(np.float32), y
    monkeypatch.setattr(o, "product_float", no_offset)
    with pytest.raises(AssertionError):
        pins.test_float_product_matches_page_decoders(o.TYPE_Q4_0)


def test_mutant_float_product_dropped_q4_k_min_is_caught(monkeypatch):
    def no_min(wtype, enc, x):
        scale, _ = o.q4_k_sub_scales(enc)
        deq = np.asarray(enc["q"], np.float64) * np.repeat(scale, 32, axis=1)
        y = np.asarray(x, np.float64) @ deq.T
        return y.astype(np.float32), y
    monkeypatch.setattr(o, "product_float", no_min)
    with pytest.raises(AssertionError):
        pins.test_float_product_matches_page_decoders(o.TYPE_Q4_K)


def test_mutant_kv_head_interleaved_is_caught(monkeypatch):
    """Query head hq reading KV head hq % n_kv instead of hq // group."""
    def interleaved(wtype, k, q, n_head):
        k = np.asarray(k, np.float32)
        n_kv, n_tok, _ = k.shape
        aq, da, sa = o.quantize_act(q)
        y = np.zeros((n_head, n_tok), np.float64)
        for hq in range(n_head):
            _, enc = o.encode_weights(wtype, k[hq % n_kv])
            y[hq] = o.product(wtype, enc, (aq[hq:hq + 1], da[hq:hq + 1], sa[hq:hq + 1]))[1][0]
        return y.astype(np.float32), y
    monkeypatch.setattr(o, "kv_scores", interleaved)
    with pytest.raises(AssertionError):
        pins.test_kv_scores_group_structure()


def _bump_codes(monkeypatch, field):
    """quantize_q4_k choosing a code one larger than needed wherever it can
    (a larger code still covers the sub-block, so the round-trip bound
    relative to the chosen scale still holds)."""
    orig = o.quantize_q4_k

    def mutant(w):
        enc = orig(w)
        c = enc[field]
        enc[field] = np.where((c > 0) & (c < 63), c + 1, c)
        # codes re-taken against the changed scale and zero point, as an
        # encoder making this choice would ([P2] §5.2 step)
        x = np.asarray(w, np.float64).reshape(enc["sc"].shape + (32,))
        S = enc["sc"] * o.f16_bits_to_f64(enc["d_bits"])[..., None]
        M = -enc["mn"] * o.f16_bits_to_f64(enc["dmin_bits"])[..., None]
        q = np.clip(o.round_half_away((x + M[..., None]) / np.where(S == 0, 1, S)[..., None]), 0, 15)
        enc["q"] = np.where((S == 0)[..., None], 0, q).astype(np.int64).reshape(enc["q"].shape)
        return enc
    monkeypatch.setattr(o, "quantize_q4_k", mutant)


def test_mutant_q4_k_scale_code_one_too_large_is_caught(monkeypatch):
    _bump_codes(monkeypatch, "sc")
    inv.test_q4_k_round_trip_bound_and_ranges()      # not caught by the bound
    with pytest.raises(AssertionError):
        inv.test_q4_k_codes_are_the_smallest_covering_ones()


def test_mutant_q4_k_min_code_one_too_large_is_caught(monkeypatch):
    _bump_codes(monkeypatch, "mn")
    with pytest.raises(AssertionError):
        inv.test_q4_k_codes_are_the_smallest_covering_ones()


@pytest.mark.parametrize("right,wrong", [(945, 900), (63, 60)])
def test_mutant_q4_k_super_block_divisor_is_caught(monkeypatch, right, wrong):
    """d from max t_j / (15 * 60) instead of / (15 * 63), or d_min from
    max m_j / 60 instead of / 63: larger super-block scales that still cover
    every sub-block."""
    orig = o.f16_ceil_div
    monkeypatch.setattr(o, "f16_ceil_div", lambda v, c: orig(v, wrong if c == right else c))
    inv.test_q4_k_round_trip_bound_and_ranges()      # not caught by the bound
    with pytest.raises(AssertionError):
        inv.test_q4_k_codes_are_the_smallest_covering_ones()
    with pytest.raises(AssertionError):
        inv.test_q4_k_hand_computed_super_block()
