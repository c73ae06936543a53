"""Pins of the oracle against what the pages print and against library
routines / brute force. CPU only."""

import json
import os
import struct
from decimal import Decimal, ROUND_HALF_UP

import numpy as np
import pytest

from oracle import qblk_oracle as o

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


# ---------------------------------------------------------------- worked examples

def test_worked_example_block_scale_0_08():
    """tech-blog page, 量化是怎么做到的？: round(x / 0.08) and codes * 0.08."""
    g = _golden("p4_worked_example.json")
    x = np.array(g["weights"], dtype=np.float32)
    s = np.float32(g["scale"])
    codes = o.round_half_away((x / s).astype(np.float64))
    assert codes.tolist() == g["codes"]
    q = np.zeros(32, dtype=np.int64)
    q[:4] = g["codes"]
    rec = o.dequant_symmetric(q[None, :], np.array([[s]], np.float32))[0, :4]
    assert np.allclose(rec, g["reconstructed"], rtol=0, atol=1e-7)


def test_q4_0_example_symmetric_rule():
    """runguoli page §5.1 example: scale 0.5, Q = [1,-2,2,7,-1]."""
    g = _golden("p2_q4_0_example.json")
    x = np.zeros((1, 32), dtype=np.float32)
    x[0, :5] = g["weights"]
    q, d = o.quantize_q4_0(x)
    assert float(d[0, 0]) == g["scale"]
    assert q[0, :5].tolist() == g["codes"]
    assert np.all(q[0, 5:] == 0)
    rec = o.dequant_symmetric(q, d)[0, :5]
    assert rec.tolist() == g["reconstructed"]
    err = np.abs(x[0, :5].astype(np.float64) - rec)
    assert np.allclose(err, g["error_magnitudes"], rtol=0, atol=1e-6)


def test_bits_per_weight_closed_forms():
    """runguoli page §5.3-§5.5 field lists; totals recomputed with the
    library's field widths (fp32 Q4_0 scale, 6-bit Q4_K codes)."""
    g = _golden("p2_bits_per_weight.json")
    for key in ("q4_0", "q8_0", "q4_k"):
        e = g[key]
        assert sum(e["fields"].values()) == e["total_bits"]
        assert e["total_bits"] / e["block"] == e["bpw"]
    K = 4096
    q40 = dict(g["q4_0"]["fields"], scale=32)
    assert o.row_bytes(o.TYPE_Q4_0, K) * 8 == sum(q40.values()) * K // 32
    assert o.row_bytes(o.TYPE_Q8_0, K) * 8 == g["q8_0"]["total_bits"] * K // 32
    q4k = dict(g["q4_k"]["fields"], scales=48, mins=48)
    assert o.row_bytes(o.TYPE_Q4_K, K) * 8 == sum(q4k.values()) * K // 256
    assert o.row_bytes(o.TYPE_Q4_K, K) / K * 8 == 4.5
    # activation buffer: 8-bit codes + fp32 scale + int32 sum per 32
    assert o.act_bytes(3, K) * 8 == 3 * K * (8 + 64 / 32)
    # the page's own Q4_0 block (fp16 scale): exactly its 144 bits, 4.5 bpw
    assert o.row_bytes(o.TYPE_Q4_0_F16, K) * 8 == g["q4_0"]["total_bits"] * K // 32
    assert o.row_bytes(o.TYPE_Q4_0_F16, K) * 8 / K == g["q4_0"]["bpw"]


def test_q4_0_f16_example_symmetric_rule():
    """runguoli page §5.1 example under the page's fp16-scale Q4_0 (§5.3):
    scale 0.5 is an fp16 value, so the codes and reconstruction are the
    printed ones."""
    g = _golden("p2_q4_0_example.json")
    x = np.zeros((1, 32), dtype=np.float32)
    x[0, :5] = g["weights"]
    q, d = o.quantize_q4_0_f16(x)
    assert float(d[0, 0]) == g["scale"]
    assert q[0, :5].tolist() == g["codes"]
    assert o.dequant_symmetric(q, d)[0, :5].tolist() == g["reconstructed"]


def _struct_half(v):
    """Nearest binary16 of a float by the standard library's IEEE half
    conversion (ties to even); OverflowError beyond the fp16 range."""
    return struct.unpack("<e", struct.pack("<e", float(v)))[0]


def test_q4_0_f16_scale_is_nearest_half_of_amax_over_7():
    rng = np.random.default_rng(5)
    w = (rng.standard_normal((64, 32 * 16)) * 10.0 ** rng.uniform(-6, 3, (64, 1))).astype(np.float32)
    q, d = o.quantize_q4_0_f16(w)
    amax = np.max(np.abs(w.reshape(64, 16, 32)), axis=-1)
    for r in range(64):
        for b in range(16):
            d32 = np.float32(amax[r, b]) / np.float32(7)
            try:
                ref = _struct_half(d32)
            except OverflowError:
                ref = 65504.0
            assert float(d[r, b]) == ref
    # saturation and an all-zero block
    big = np.zeros((1, 64), dtype=np.float32)
    big[0, 0] = 1e6
    qb, db = o.quantize_q4_0_f16(big)
    assert float(db[0, 0]) == 65504.0 and qb[0, 0] == 7
    assert float(db[0, 1]) == 0.0 and np.all(qb[0, 32:] == 0)


# ---------------------------------------------------------------- scalar kernel of §6.4

def _page_q4_0_scalar_dot(scales, qs, yf):
    """The scalar Q4_0 dot of runguoli page §6.4, restated once for both scale
    widths: for every block, take its scale; for every byte j of the block,
    low nibble - 8 pairs with float activation 2j and high nibble - 8 with
    2j+1; accumulate (code * scale) * activation."""
    total = 0.0
    for blk in range(len(scales)):
        scale = float(scales[blk])
        for j in range(16):
            byte = int(qs[16 * blk + j])
            lo = (byte & 0x0F) - 8
            hi = (byte >> 4) - 8
            total += (lo * scale) * float(yf[32 * blk + 2 * j])
            total += (hi * scale) * float(yf[32 * blk + 2 * j + 1])
    return total


def _page_q4_0_float_dot(packed_row, K, yf):
    """The page's scalar kernel on the library's Q4_0 row (fp32 scales)."""
    nb = K // 32
    scales = packed_row[:4 * nb].copy().view("<f4")
    return _page_q4_0_scalar_dot(scales, packed_row[o.header_bytes(o.TYPE_Q4_0, K):], yf)


def test_q4_0_pack_matches_page_scalar_kernel():
    rng = np.random.default_rng(11)
    K = 256
    w = (rng.standard_normal((3, K)) * 0.02).astype(np.float32)
    yf = rng.standard_normal(K)
    packed, enc = o.encode_weights(o.TYPE_Q4_0, w)
    deq = o.dequant_weights(o.TYPE_Q4_0, enc)
    for n in range(3):
        ref = float(deq[n] @ yf)
        got = _page_q4_0_float_dot(packed[n], K, yf)
        assert abs(got - ref) <= 1e-12 * max(1.0, abs(ref))


def test_q4_0_f16_pack_matches_page_scalar_kernel():
    """The same scalar kernel reading fp16 scales: the page's 18-byte block."""
    rng = np.random.default_rng(12)
    K = 256
    w = (rng.standard_normal((3, K)) * 0.02).astype(np.float32)
    yf = rng.standard_normal(K)
    packed, enc = o.encode_weights(o.TYPE_Q4_0_F16, w)
    deq = o.dequant_weights(o.TYPE_Q4_0_F16, enc)
    for n in range(3):
        total = _page_q4_0_f16_float_dot(packed[n], K, yf)
        ref = float(deq[n] @ yf)
        assert abs(total - ref) <= 1e-12 * max(1.0, abs(ref))


def test_q4_0_pack_nibble_order_is_pinned():
    """A block whose codes differ between even and odd positions: swapping the
    nibble order would change the page-kernel result."""
    K = 32
    x = np.zeros((1, K), dtype=np.float32)
    x[0, 0::2] = 0.7
    x[0, 1::2] = -0.1
    x[0, 1] = -0.7
    packed, enc = o.encode_weights(o.TYPE_Q4_0, x)
    yf = np.zeros(K)
    yf[0] = 1.0
    got = _page_q4_0_float_dot(packed[0], K, yf)
    assert got == pytest.approx(0.7, abs=1e-7)
    yf[:] = 0
    yf[1] = 1.0
    assert _page_q4_0_float_dot(packed[0], K, yf) == pytest.approx(-0.7, abs=1e-7)


# ---------------------------------------------------------------- helpers vs library routines

def test_round_half_away_matches_decimal():
    vals = [0.5, 1.5, 2.5, -0.5, -1.5, -2.5, 0.49999997, -0.49999997, 126.5,
            -126.5, 3.4999998, 7.5, -7.5, 0.0, -0.0, 1e-30, 127.0, 2.0 ** 40 + 0.5]
    rng = np.random.default_rng(3)
    vals += list(rng.uniform(-130, 130, 2000))
    vals += list(np.round(rng.uniform(-130, 130, 200)) + 0.5)
    got = o.round_half_away(np.array(vals, dtype=np.float64))
    for v, g in zip(vals, got):
        ref = float(Decimal(float(v)).quantize(Decimal(1), rounding=ROUND_HALF_UP))
        assert g == ref, (v, g, ref)


def test_f16_decode_matches_numpy_half():
    bits = np.arange(0, 0x7C00, dtype=np.int64)
    bits = np.concatenate([bits, bits | 0x8000])
    ref = bits.astype(np.uint16).view(np.float16).astype(np.float64)
    got = o.f16_bits_to_f64(bits)
    assert np.array_equal(got, ref)


def test_f16_ceil_div_brute_force():
    allbits = np.arange(0, 0x7C00, dtype=np.int64)
    allvals = allbits.astype(np.uint16).view(np.float16).astype(np.float64)
    rng = np.random.default_rng(5)
    for c in (63, 945):
        v = np.concatenate([
            [0.0, 5.9604645e-08 * c, 1e-12, 1.0, c * 65504.0],
            rng.uniform(0, 1, 300) ** 4 * 3.0,
            allvals[rng.integers(1, len(allvals), 100)] * c,   # exact hits
        ])
        got = o.f16_ceil_div(v, c)
        for vi, gi in zip(v, got):
            ok = np.nonzero(c * allvals >= vi)[0]
            assert gi == allbits[ok[0]], (c, vi)


# ---------------------------------------------------------------- float-activation product

def _page_q4_0_f16_float_dot(packed_row, K, yf):
    """The page's scalar kernel reading the page's fp16 scales."""
    nb = K // 32
    scales = packed_row[:2 * nb].copy().view("<f2")
    return _page_q4_0_scalar_dot(scales, packed_row[o.header_bytes(o.TYPE_Q4_0_F16, K):], yf)


def _page_q8_0_float_dot(packed_row, K, yf):
    """Q8_0 (runguoli page §5.4: one fp32 scale, 32 int8 per block) decoded
    from the library's row: the 8 codes of each group are stored as elements
    0,2,4,6,1,3,5,7."""
    nb = K // 32
    scales = packed_row[:4 * nb].copy().view("<f4")
    qs = packed_row[o.header_bytes(o.TYPE_Q8_0, K):].copy().view(np.int8)
    order = (0, 2, 4, 6, 1, 3, 5, 7)
    total = 0.0
    for blk in range(nb):
        for p in range(32):
            g, pos = divmod(p, 8)
            total += (int(qs[32 * blk + p]) * float(scales[blk])) * float(yf[32 * blk + 8 * g + order[pos]])
    return total


def _page_q4_k_float_dot(packed_row, K, yf):
    """Q4_K (runguoli page §5.5: weight = q * (d * scale_j) + d_min * min_j)
    decoded from the library's row: per super-block a header of fp16 d, fp16
    d_min and a 96-bit field with 6-bit sc_j at bit 6j and mn_j at bit
    48 + 6j, then 8 x 16 bytes whose byte t of sub-block j holds elements 2t
    (low nibble) and 2t + 1 (high nibble)."""
    nsb = K // 256
    hdr = packed_row[:16 * nsb]
    qs = packed_row[16 * nsb:]
    total = 0.0
    for sb in range(nsb):
        h = hdr[16 * sb:16 * sb + 16]
        d = float(h[0:2].copy().view("<f2")[0])
        dmin = float(h[2:4].copy().view("<f2")[0])
        field = int.from_bytes(bytes(h[4:16]), "little")
        for j in range(8):
            sc = (field >> (6 * j)) & 63
            mn = (field >> (48 + 6 * j)) & 63
            for t in range(16):
                byte = int(qs[128 * sb + 16 * j + t])
                for e, q in ((2 * t, byte & 0x0F), (2 * t + 1, byte >> 4)):
                    total += (q * (d * sc) + dmin * mn) * float(yf[256 * sb + 32 * j + e])
    return total


_PAGE_FLOAT_DOT = {o.TYPE_Q4_0: _page_q4_0_float_dot, o.TYPE_Q8_0: _page_q8_0_float_dot,
                   o.TYPE_Q4_K: _page_q4_k_float_dot, o.TYPE_Q4_0_F16: _page_q4_0_f16_float_dot}


@pytest.mark.parametrize("wtype", [o.TYPE_Q4_0, o.TYPE_Q8_0, o.TYPE_Q4_K, o.TYPE_Q4_0_F16])
def test_float_product_matches_page_decoders(wtype):
    """product_float against the pages' decoders restated over the packed
    bytes, element by element (no shared code with the oracle's unpackers)."""
    rng = np.random.default_rng(60 + wtype)
    N, M, K = 3, 2, 512
    w = (rng.standard_normal((N, K)) * 0.02).astype(np.float32)
    w[0, 40:80] = np.abs(w[0, 40:80])  # a sub-block with a zero point of 0
    x = rng.standard_normal((M, K)).astype(np.float32)
    packed, enc = o.encode_weights(wtype, w)
    y32, y64 = o.product_float(wtype, enc, x)
    assert y64.shape == (M, N)
    for m in range(M):
        for n in range(N):
            ref = _PAGE_FLOAT_DOT[wtype](packed[n], K, x[m].astype(np.float64))
            assert abs(y64[m, n] - ref) <= 1e-12 * max(1.0, abs(ref))
            assert y32[m, n] == np.float32(y64[m, n])


@pytest.mark.parametrize("wtype", [o.TYPE_Q4_0, o.TYPE_Q8_0, o.TYPE_Q4_K, o.TYPE_Q4_0_F16])
def test_float_product_on_dequantized_activations_is_the_quantized_product(wtype):
    """With x = the dequantized Q8 activations (exact in fp64), the float
    product and the integer-block product are the same sum, regrouped."""
    rng = np.random.default_rng(70 + wtype)
    N, M, K = 5, 3, 768
    w = (rng.standard_normal((N, K)) * 0.02).astype(np.float32)
    x = rng.standard_normal((M, K)).astype(np.float32)
    _, enc = o.encode_weights(wtype, w)
    aq, da, sa = o.quantize_act(x)
    xdeq = np.asarray(aq, np.float64) * np.repeat(np.asarray(da, np.float64), 32, axis=1)
    yf = o.product_float(wtype, enc, xdeq)[1]
    yq = o.product(wtype, enc, (aq, da, sa))[1]
    assert np.max(np.abs(yf - yq)) <= 1e-12 * np.max(np.abs(yq))


def test_float_product_unit_activation_picks_a_weight_column():
    """x = e_k gives column k of the decoded weights, for every k of a block
    (catches a transposed or shifted activation index)."""
    rng = np.random.default_rng(80)
    K = 256
    w = (rng.standard_normal((2, K)) * 0.02).astype(np.float32)
    packed, enc = o.encode_weights(o.TYPE_Q4_K, w)
    deq = o.dequant_weights(o.TYPE_Q4_K, enc)
    for kk in (0, 1, 31, 32, 255):
        x = np.zeros((1, K), np.float32)
        x[0, kk] = 1.0
        assert np.array_equal(o.product_float(o.TYPE_Q4_K, enc, x)[1][0], deq[:, kk])
        assert _page_q4_k_float_dot(packed[1], K, x[0].astype(np.float64)) == deq[1, kk]


# ---------------------------------------------------------------- quantized KV cache

@pytest.mark.parametrize("wtype", [o.TYPE_Q4_0, o.TYPE_Q8_0, o.TYPE_Q4_0_F16])
def test_kv_scores_match_page_decoders_with_grouped_heads(wtype):
    """Each score is the pages' decoded key row times the dequantized query
    (exact in fp64), with query head hq reading KV head hq // group."""
    rng = np.random.default_rng(100 + wtype)
    n_kv, n_head, n_tok, hd = 2, 6, 5, 64
    k = rng.standard_normal((n_kv, n_tok, hd)).astype(np.float32)
    q = rng.standard_normal((n_head, hd)).astype(np.float32)
    y32, y64 = o.kv_scores(wtype, k, q, n_head)
    assert y64.shape == (n_head, n_tok)
    aq, da, _ = o.quantize_act(q)
    qdeq = np.asarray(aq, np.float64) * np.repeat(np.asarray(da, np.float64), 32, axis=1)
    for hq in range(n_head):
        packed, _ = o.encode_weights(wtype, k[hq // 3])
        for t in range(n_tok):
            ref = _PAGE_FLOAT_DOT[wtype](packed[t], hd, qdeq[hq])
            assert abs(y64[hq, t] - ref) <= 1e-12 * max(1.0, abs(ref))


def test_kv_scores_group_structure():
    """Equal queries in one group give equal rows; a zero KV head gives zero
    scores for exactly its group."""
    rng = np.random.default_rng(110)
    n_kv, n_head, n_tok, hd = 2, 8, 7, 128
    k = rng.standard_normal((n_kv, n_tok, hd)).astype(np.float32)
    k[1] = 0.0
    q = np.repeat(rng.standard_normal((1, hd)).astype(np.float32), n_head, axis=0)
    y = o.kv_scores(o.TYPE_Q8_0, k, q, n_head)[1]
    assert np.all(y[:4] == y[0]) and np.any(y[0] != 0.0)
    assert np.all(y[4:] == 0.0)
