"""Invariants and brute-force pins of the oracle. CPU only."""

import numpy as np
import pytest

from oracle import qblk_oracle as o

TYPES = [o.TYPE_Q4_0, o.TYPE_Q8_0, o.TYPE_Q4_K, o.TYPE_Q4_0_F16]


def _blocks_with_special_cases(rng, rows, K, std=0.02):
    """Seeded rows with zero, constant, single-non-zero and outlier blocks."""
    w = (rng.standard_normal((rows, K)) * std).astype(np.float32)
    w[0, 0:32] = 0.0                      # all-zero block
    w[0, 32:64] = 0.013                   # constant positive block
    w[0, 64:96] = -0.021                  # constant negative block
    w[0, 96:128] = 0.0
    w[0, 100] = -0.05                     # single non-zero
    if K >= 512:
        w[1, 256:512] = 0.0               # all-zero super-block
        w[1, 512 - 32:512] = 0.0
    idx = rng.choice(rows * K, size=max(1, rows * K // 1000), replace=False)
    w.reshape(-1)[idx] = np.where(rng.random(idx.size) < 0.5, -1, 1) * 10 * std
    return w


# ---------------------------------------------------------------- round trip

@pytest.mark.parametrize("qmax", [7, 127])
def test_symmetric_round_trip_bound(qmax):
    """|x - Q*scale| <= scale/2 per block ([P2] §5.1), up to the fp32 rounding
    of x/scale: |x/scale - fl(x/scale)| <= qmax * 2^-24."""
    rng = np.random.default_rng(100 + qmax)
    w = _blocks_with_special_cases(rng, 64, 1024)
    q, d = o.quantize_symmetric(w, qmax)
    assert q.min() >= -qmax and q.max() <= qmax
    rec = o.dequant_symmetric(q, d)
    err = np.abs(w.astype(np.float64) - rec).reshape(64, -1, 32).max(-1)
    bound = d.astype(np.float64) * (0.5 + qmax * 2.0 ** -24)
    assert np.all(err <= bound)
    # the bound is not vacuous: most blocks use more than half of it
    assert np.mean(err > 0.25 * d) > 0.5


def test_symmetric_special_blocks():
    x = np.zeros((4, 32), dtype=np.float32)
    x[1, 5] = -0.3                  # single non-zero -> exactly -qmax
    x[2, :] = 0.25                  # constant block
    x[3, :] = np.linspace(-1, 1, 32)
    for qmax in (7, 127):
        q, d = o.quantize_symmetric(x, qmax)
        assert d[0] == 0 and np.all(q[0] == 0)
        assert q[1, 5] == -qmax and np.count_nonzero(q[1]) == 1
        assert np.all(q[2] == qmax)
        assert q[3, 0] == -qmax and q[3, -1] == qmax
        rec = o.dequant_symmetric(q, d)
        assert abs(rec[1, 5] + 0.3) <= 1e-7
        assert np.allclose(rec[2], 0.25, atol=1e-7)
    q, d = o.quantize_q4_0(x[:1])
    packed = o.pack_q4_0(q, d)
    assert np.all(packed[0, o.header_bytes(o.TYPE_Q4_0, 32):] == 0x88)


def test_q4_k_round_trip_bound_and_ranges():
    """|x - x^| <= scale_j / 2 per sub-block for the [P2] §5.5 dequant."""
    rng = np.random.default_rng(7)
    w = _blocks_with_special_cases(rng, 48, 2048)
    enc = o.quantize_q4_k(w)
    assert enc["q"].min() >= 0 and enc["q"].max() <= 15
    assert enc["sc"].min() >= 0 and enc["sc"].max() <= 63
    assert enc["mn"].min() >= 0 and enc["mn"].max() <= 63
    assert np.all(o.f16_bits_to_f64(enc["dmin_bits"]) <= 0)
    assert np.all(o.f16_bits_to_f64(enc["d_bits"]) >= 0)
    rec = o.dequant_q4_k(enc)
    scale, mins = o.q4_k_sub_scales(enc)
    err = np.abs(w.astype(np.float64) - rec).reshape(48, -1, 32).max(-1)
    assert np.all(err <= scale * 0.5 * (1 + 1e-12))
    # zero sub-blocks reconstruct exactly
    assert np.all(rec[1, 256:512] == 0)
    assert np.all(rec[0, 0:32] == 0)
    # constant sub-blocks reconstruct within half a step
    assert np.allclose(rec[0, 32:64], 0.013, atol=float(scale[0, 1]) / 2 + 1e-12)


def test_q4_k_all_positive_and_all_negative_super_blocks():
    rng = np.random.default_rng(8)
    w = np.abs(rng.standard_normal((2, 256))).astype(np.float32)
    w[1] = -w[1]
    enc = o.quantize_q4_k(w)
    assert enc["dmin_bits"][0, 0] == 0 and np.all(enc["mn"][0] == 0)
    assert np.all(enc["mn"][1] > 0)
    rec = o.dequant_q4_k(enc)
    scale, _ = o.q4_k_sub_scales(enc)
    err = np.abs(w - rec).reshape(2, 8, 32).max(-1)
    assert np.all(err <= scale * 0.5 * (1 + 1e-12))


def test_q4_k_hand_built_block_dequant():
    """[P2] §5.5: x^[32j+i] = qs * (d * scales[j]) + d_min * mins[j], on a
    hand-built super-block: d = 0.5 (fp16 0x3800), d_min = -0.25 (0xB400),
    scales[j] = j + 1, mins[j] = 2j, qs[32j + i] = i % 16."""
    enc = dict(d_bits=np.array([[0x3800]], np.uint16),
               dmin_bits=np.array([[0xB400]], np.uint16),
               sc=np.arange(1, 9, dtype=np.int64)[None, None, :],
               mn=(2 * np.arange(8, dtype=np.int64))[None, None, :],
               q=(np.arange(256) % 16)[None, :].astype(np.int64))
    rec = o.dequant_q4_k(enc)[0]
    # values worked out by hand
    assert rec[0] == 0.0                         # j=0: 0*0.5 + 0
    assert rec[5] == 2.5                         # j=0: 5*0.5
    assert rec[32 + 3] == 3 * 1.0 - 0.5          # j=1: scale 1.0, min -0.5
    assert rec[7 * 32 + 15] == 15 * 4.0 - 3.5    # j=7: scale 4.0, min -3.5
    assert rec[7 * 32 + 16] == 0 * 4.0 - 3.5


def test_q4_k_header_bit_layout():
    """Header layout: d, d_min as fp16, then a 96-bit little-endian field,
    sc_j at bit 6j and mn_j at bit 48 + 6j. Checked by building the expected
    bytes from a string of bits."""
    rng = np.random.default_rng(9)
    sc = rng.integers(0, 64, (1, 1, 8))
    mn = rng.integers(0, 64, (1, 1, 8))
    enc = dict(d_bits=np.array([[0x1234]], np.uint16),
               dmin_bits=np.array([[0x8765]], np.uint16),
               sc=sc, mn=mn, q=np.zeros((1, 256), np.int64))
    packed = o.pack_q4_k(enc)[0]
    assert packed[0] == 0x34 and packed[1] == 0x12
    assert packed[2] == 0x65 and packed[3] == 0x87
    bits = ""                                   # bit i of the field = bits[i]
    for v in list(sc[0, 0]) + list(mn[0, 0]):
        bits += format(int(v), "06b")[::-1]
    expect = [int(bits[8 * b:8 * b + 8][::-1], 2) for b in range(12)]
    assert packed[4:16].tolist() == expect
    back = o.unpack_q4_k(packed[None, :], 256)
    assert np.array_equal(back["sc"], sc) and np.array_equal(back["mn"], mn)


def test_q4_k_nibble_layout():
    q = (np.arange(256) * 7 % 16)[None, :].astype(np.int64)
    enc = dict(d_bits=np.zeros((1, 1), np.uint16),
               dmin_bits=np.zeros((1, 1), np.uint16),
               sc=np.zeros((1, 1, 8), np.int64), mn=np.zeros((1, 1, 8), np.int64), q=q)
    packed = o.pack_q4_k(enc)[0]
    for j in range(8):
        for t in range(16):
            byte = packed[16 + 16 * j + t]
            assert byte & 15 == q[0, 32 * j + 2 * t]
            assert byte >> 4 == q[0, 32 * j + 2 * t + 1]


def test_activation_buffer_layout():
    x = np.zeros((2, 64), dtype=np.float32)
    x[0, :32] = np.arange(32) - 16
    x[0, 32:] = 127.0
    x[1, 5] = 1.0
    q, d, s = o.quantize_act(x)
    buf = o.pack_act(q, d, s)
    assert buf.size == o.act_bytes(2, 64)
    codes = buf[:128].view(np.int8)
    # first group of 8 elements stored as 0,2,4,6,1,3,5,7
    assert codes[:8].tolist() == [q[0, i] for i in (0, 2, 4, 6, 1, 3, 5, 7)]
    ds = buf[128:].view("<u4").reshape(2, 2, 2)
    assert ds[0, 0, 0].view("<f4") == np.float32(16) / np.float32(127)
    assert ds[0, 0, 1].view("<i4") == q[0, :32].sum()
    assert ds[0, 1, 1].view("<i4") == 32 * 127
    assert ds[1, 0, 1].view("<i4") == 127 and ds[1, 1, 0] == 0
    back = o.unpack_act(buf, 2, 64)
    for a, b in zip((q, d, s), back):
        assert np.array_equal(a, b)


@pytest.mark.parametrize("wtype", TYPES)
def test_pack_unpack_round_trip(wtype):
    rng = np.random.default_rng(20 + wtype)
    w = _blocks_with_special_cases(rng, 5, 512)
    packed, enc = o.encode_weights(wtype, w)
    assert packed.shape == (5, o.row_bytes(wtype, 512))
    if wtype == o.TYPE_Q4_K:
        back = o.unpack_q4_k(packed, 512)
        for k in enc:
            assert np.array_equal(back[k], enc[k]), k
    else:
        unpack = {o.TYPE_Q4_0: o.unpack_q4_0, o.TYPE_Q8_0: o.unpack_q8_0,
                  o.TYPE_Q4_0_F16: o.unpack_q4_0_f16}[wtype]
        q, d = unpack(packed, 512)
        assert np.array_equal(q, enc["q"]) and np.array_equal(d, enc["d"])


# ---------------------------------------------------------------- integer block sums

def _brute_block_sums(wq, aq):
    N, K = len(wq), len(wq[0])
    M = len(aq)
    out = [[[0] * (K // 32) for _ in range(N)] for _ in range(M)]
    for m in range(M):
        for n in range(N):
            for b in range(K // 32):
                acc = 0
                for i in range(32 * b, 32 * b + 32):
                    acc += int(wq[n][i]) * int(aq[m][i])
                out[m][n][b] = acc
    return out


@pytest.mark.parametrize("wtype", TYPES)
@pytest.mark.parametrize("N,K,M", [(1, 256, 1), (2, 512, 2), (3, 256, 5), (7, 512, 1)])
def test_block_sums_brute_force(wtype, N, K, M):
    rng = np.random.default_rng(1000 * wtype + 17 * N + M)
    w = _blocks_with_special_cases(rng, max(N, 2), K)[:N]
    x = rng.standard_normal((M, K)).astype(np.float32)
    _, enc = o.encode_weights(wtype, w)
    aq, da, sa = o.quantize_act(x)
    wq = o.weight_codes_for_sums(wtype, enc)
    got = o.block_sums(wq, aq)
    ref = _brute_block_sums(wq.tolist(), aq.tolist())
    assert got.tolist() == ref
    # the activation block sums
    assert sa.tolist() == [[sum(aq[m, 32 * b:32 * b + 32].tolist()) for b in range(K // 32)]
                           for m in range(M)]


@pytest.mark.parametrize("K", [32, 64])
def test_block_sums_small_k_symmetric(K):
    rng = np.random.default_rng(K)
    w = rng.standard_normal((3, K)).astype(np.float32)
    x = rng.standard_normal((2, K)).astype(np.float32)
    for wtype in (o.TYPE_Q4_0, o.TYPE_Q8_0, o.TYPE_Q4_0_F16):
        _, enc = o.encode_weights(wtype, w)
        aq, _, _ = o.quantize_act(x)
        assert o.block_sums(enc["q"], aq).tolist() == _brute_block_sums(
            enc["q"].tolist(), aq.tolist())


# ---------------------------------------------------------------- float result

@pytest.mark.parametrize("wtype", TYPES)
def test_product_equals_dequantized_dot(wtype):
    """The regrouped integer product equals the fp64 dot product of the
    dequantized operands."""
    rng = np.random.default_rng(300 + wtype)
    N, K, M = 37, 1024, 6
    w = _blocks_with_special_cases(rng, N, K)
    x = rng.standard_normal((M, K)).astype(np.float32)
    _, enc = o.encode_weights(wtype, w)
    act = o.quantize_act(x)
    y32, y64 = o.product(wtype, enc, act)
    ref = o.dequant_dot(o.dequant_weights(wtype, enc),
                        o.dequant_symmetric(act[0], act[1]))
    assert o.rel_err(y64, ref) <= 1e-12
    assert np.array_equal(y32, y64.astype(np.float32))
    # and close to the unquantized product (quantization error only)
    exact = x.astype(np.float64) @ w.astype(np.float64).T
    assert o.rel_err(y64, exact) < 0.2


def test_power_of_two_scales_product_is_exact():
    """With power-of-two scales and small codes every fp64 step is exact, so
    y equals the integer result times the scale."""
    rng = np.random.default_rng(4)
    K = 512
    q = rng.integers(-7, 8, (4, K))
    d = np.full((4, K // 32), 2.0 ** -6, np.float32)
    xi = rng.integers(-127, 128, (3, K))
    xi[:, ::32] = 127
    x = (xi * 2.0 ** -3).astype(np.float32)
    aq, da, sa = o.quantize_act(x)
    assert np.array_equal(aq, xi) and np.all(da == 2.0 ** -3)
    y32, y64 = o.product_sym(q, d, aq, da)
    ref = (xi @ q.T) * 2.0 ** -9
    assert np.array_equal(y64, ref)


def test_q4_0_f16_round_trip_bound_and_ranges():
    """Codes in [-7, 7] against the stored fp16 scale, |x - q*d16| <= d16/2
    (the fp32 quotient's rounding aside), blocks with outliers included."""
    rng = np.random.default_rng(31)
    w = _blocks_with_special_cases(rng, 16, 1024)
    q, d = o.quantize_q4_0_f16(w)
    assert q.min() >= -7 and q.max() <= 7
    rec = o.dequant_symmetric(q, d)
    err = np.abs(w.astype(np.float64) - rec).reshape(16, 32, 32)
    bound = np.asarray(d, np.float64)[..., None] * (0.5 + 1e-6)
    assert np.all(err <= bound)
    # the stored scale is an fp16 value
    assert np.array_equal(np.asarray(d).astype(np.float16).astype(np.float32), d)


# ---------------------------------------------------------------- Q4_K code choices (reading R8)

def _f16_value(bits):
    """fp16 bit patterns -> fp64 values, through NumPy's own binary16 type."""
    return np.asarray(bits, np.uint16).view(np.float16).astype(np.float64)


def _f16_prev(bits):
    """The next smaller fp16 value of non-negative, non-zero patterns: the
    bit pattern stepped down by one."""
    return _f16_value(np.asarray(bits, np.int64) - 1)


def _q4_k_minimality(w, enc):
    """Checks the R8 choices of one encoding against the raw fp32 rows:
    every code and super-block scale covers its sub-block ([P2] §5.2 range
    hi - lo split into 15 steps, zero point -M_j <= lo_j) and is the smallest
    one that does. Recomputes m_j, hi_j and t_j from the input, not from the
    oracle's intermediate values."""
    x = np.asarray(w, np.float64)
    N, K = x.shape
    xs = x.reshape(N, K // 256, 8, 32)
    hi = xs.max(-1)
    m = np.maximum(0.0, -xs.min(-1))
    dmp_bits = np.asarray(enc["dmin_bits"], np.int64) & 0x7FFF
    dmp = _f16_value(dmp_bits)
    d_bits = np.asarray(enc["d_bits"], np.int64)
    d = _f16_value(d_bits)
    sc, mn = enc["sc"], enc["mn"]
    mmax = m.max(-1)
    # d_min: covers (63 * dmin+ >= max m_j), and one fp16 step less does not
    assert np.all(63 * dmp >= mmax)
    pos = dmp_bits > 0
    assert np.all(63 * _f16_prev(np.where(pos, dmp_bits, 1))[pos] < mmax[pos])
    assert np.all(mmax[~pos] == 0)
    # mn_j: covers, and mn_j - 1 does not
    Mj = mn * dmp[..., None]
    assert np.all(Mj >= m)
    assert np.all(((mn - 1) * dmp[..., None] < m)[mn > 0])
    assert np.all(mn[m == 0] == 0)
    # d: 945 d >= max t_j with t_j = hi_j + M_j, and one fp16 step less does not
    t = hi + Mj
    tmax = t.max(-1)
    assert np.all(945 * d >= tmax)
    dp = d_bits > 0
    assert np.all(945 * _f16_prev(np.where(dp, d_bits, 1))[dp] < tmax[dp])
    assert np.all(tmax[~dp] <= 0)
    # sc_j: covers (15 sc_j d >= t_j), and sc_j - 1 does not
    assert np.all(15 * sc * d[..., None] >= t)
    assert np.all((15 * (sc - 1) * d[..., None] < t)[sc > 0])


def _minimality_inputs():
    rng = np.random.default_rng(71)
    sets = [_blocks_with_special_cases(rng, 24, 2048)]
    pos = np.abs(rng.standard_normal((4, 512))).astype(np.float32) * 0.02
    sets.append(pos)                       # all-positive super-blocks
    sets.append(-pos)                      # all-negative super-blocks
    sets.append((rng.standard_t(5, (8, 1024)) * 0.02 / np.sqrt(5 / 3)).astype(np.float32))
    # ranges spanning many binades, from tiny to large super-blocks
    sets.append((rng.standard_normal((8, 256)) * np.logspace(-6, 3, 8)[:, None]).astype(np.float32))
    return sets


def test_q4_k_codes_are_the_smallest_covering_ones():
    """Reading R8 pinned directly: d_min, mn_j, d and sc_j are each the
    smallest value that covers its sub-blocks, on seeded rows with special
    blocks, all-positive and all-negative super-blocks, heavy tails and
    scales from 1e-6 to 1e3."""
    for w in _minimality_inputs():
        _q4_k_minimality(w, o.quantize_q4_k(w))


def test_q4_k_hand_computed_super_block():
    """One super-block worked out by hand from [P2] §5.2/§5.5 and reading
    R8 (tests/golden/q4_k_hand_superblock.json, derivation in its note):
    d, d_min, the 8 scale and min codes and the codes of every element."""
    import json
    import os
    g = json.load(open(os.path.join(os.path.dirname(__file__), "golden",
                                    "q4_k_hand_superblock.json")))
    w = np.zeros((1, 256), np.float32)
    for j in range(8):
        w[0, 32 * j] = g["lo"][j]
        w[0, 32 * j + 1] = g["hi"][j]
    enc = o.quantize_q4_k(w)
    assert int(enc["d_bits"][0, 0]) == g["d_bits"]
    assert int(enc["dmin_bits"][0, 0]) == g["dmin_bits"]
    assert enc["sc"][0, 0].tolist() == g["sc"]
    assert enc["mn"][0, 0].tolist() == g["mn"]
    q = enc["q"][0].reshape(8, 32)
    assert q[:, 0].tolist() == g["q_lo"]
    assert q[:, 1].tolist() == g["q_hi"]
    for j in range(8):
        assert np.all(q[j, 2:] == g["q_zero"][j]), j
    _q4_k_minimality(w, enc)
