"""Plain CPU oracle for the block-quantized weight x activation product.

TEST INFRASTRUCTURE. Only the test suite, the smoke check and the benchmark's
CPU-baseline leg may import this module. The product path (the HIP library and
its Python binding) never imports, calls or links it, and this module imports
nothing from the product path.

Everything here is deliberately slow and literal: NumPy, integer codes in
int64, floating point in fp64 except where the encoding itself fixes fp32. No
blocking, fusion or reordering beyond what the definitions below state.

Sources (web pages; cited by title and section):

* [P2] "llama.cpp 推理引擎" (runguoli.com/llm-libs/14-llama-cpp)
    - §5.1 对称量化 (symmetric quantization): Q = round(x / scale),
      scale = max|x| / (2^(b-1) - 1), dequant x^ = Q * scale.
    - §5.2 非对称量化 (asymmetric): Q = round((x - zp) / scale),
      scale = (max - min) / (2^b - 1), zp = min, x^ = Q * scale + zp.
    - §5.3 Q4_0 详解: 32-weight groups, one scale, 32 4-bit integers.
    - §5.4 Q8_0 详解: 32-weight groups, one fp32 scale, 32 int8.
    - §5.5 K-quant 数学原理: 256-weight super-block with fp16 d and d_min,
      8 sub-blocks with their own scale and min codes; dequant of element i
      of sub-block j is qs * (d * scales[j]) + d_min * mins[j].
    - §6.4 量化内核优化: the scalar Q4_0 dot kernel, which fixes the nibble
      order (low nibble = even element, high nibble = odd element) and the
      decode offset of 8; scales are applied outside the integer values.
* [P3] wmrh.cn article on llama.cpp as a "bare engine", §2.2 量化不是“压缩”
  是“计算友好型重编码”: the Q4_K x Q8 dot is an int4 x int8 integer
  multiply-add inside each block, with the float scales outside.
* [P4] "llama.cpp：一个人、一个周末、一个改变 AI 推理格局的 C++ 文件"
  (tech-blog-56a.pages.dev), section 量化是怎么做到的？: 32-weight blocks
  sharing one scale (worked example with scale 0.08) and the K-quant
  hierarchy of 256-weight super-blocks made of 8 sub-blocks of 32.

Readings where the pages are silent or disagree (numbered as in the design
notes; the ones without an effect on this module are not repeated here):

R1  Q4_0 and Q8_0 scales are fp32 (the Q4_0 page text says fp16; the workload
    being reproduced states fp32 for both).
R2  Q4_0 encodes q in [-7, 7] (scale = amax/7 per [P2] §5.1); the stored
    nibble is q + 8 and the decoder accepts the full nibble range 0..15 as
    nibble - 8 ([P2] §6.4).
R3  Activations are quantized with the [P2] §5.1 rule at b = 8, per row and
    per 32 consecutive elements, with an fp32 scale; the integer block sum
    A = sum(q) is stored beside the scale.
R4  "round" is round-half-away-from-zero; divisions are IEEE fp32 divisions
    (correctly rounded) for the fp32 encodings and IEEE fp64 for Q4_K.
R5  An all-zero block has scale 0 and all codes 0.
R6  Q4_K sub-scales and sub-mins are 6-bit codes (the page draws 4-bit; the
    workload states 6-bit). Sub-blocks are 32 wide.
R7  Q4_K zero point: the sub-block minimum, but never above 0, so that one
    super-block min scale (stored as a non-positive fp16 d_min) and unsigned
    6-bit mins can represent every sub-block: x^ = (d*sc_j)*q + d_min*mn_j.
R8  Q4_K d and d_min are the smallest fp16 values that let the 6-bit codes
    cover every sub-block, and sc_j / mn_j are the smallest codes that cover
    sub-block j; this guarantees |x - x^| <= (d*sc_j)/2 (see quantize_q4_k).
R12 [P2] §6.4's scalar kernel multiplies decoded weights by float
    activations, while the Q4_K x Q8 dot of [P3] §2.2 quantizes them: the
    hot path quantizes activations to Q8 32-blocks (R3); the float form is a
    separate product (product_float) over the same packed weights.
R18 The pages' own Q4_0 block ([P2] §5.3: one fp16 scale and 32 4-bit
    integers, 144 bits) is a second 4-bit symmetric type, Q4_0_F16: the
    scale is the fp32 amax/7 of R1/R2 rounded to the nearest fp16 (ties to
    even; values beyond the fp16 range saturate at 65504), and the codes are
    taken against that stored scale, q = round_half_away(x / d16) in fp32,
    clamped to [-7, 7], so that x^ = q * d16 is what the decoder rebuilds.

Packed byte layouts (the library's own, little-endian, described in
include/qblk.h) are produced by the pack_* functions below.
"""

import numpy as np

QK = 32           # elements per block / sub-block ([P2] §5.3, §5.4; [P4])
QK_K = 256        # elements per K-quant super-block ([P2] §5.5; [P4])
SUBS = QK_K // QK  # 8 sub-blocks per super-block ([P4])

TYPE_Q4_0 = 1
TYPE_Q8_0 = 2
TYPE_Q4_K = 3
TYPE_Q4_0_F16 = 4

# byte order of the 8 elements of a group of eight inside every int8 block of
# the activation buffer and of Q8_0 weights: even elements first, then odd
# ones. It is the order in which the two nibbles of four consecutive bytes of
# a 4-bit block come out ([P2] §6.4 nibble order), so dot products need no
# byte shuffles. A dot product over a block does not depend on this order.
GROUP8_ORDER = np.array([0, 2, 4, 6, 1, 3, 5, 7])


# --------------------------------------------------------------------------
# scalar helpers
# --------------------------------------------------------------------------

def round_half_away(v):
    """Round to nearest integer, ties away from zero (reading R4). fp64 in/out.

    Written so that it is exact for every fp64 input: floor() and v - floor(v)
    are exact in binary floating point.
    """
    v = np.asarray(v, dtype=np.float64)
    a = np.abs(v)
    r = np.floor(a)
    r = r + ((a - r) >= 0.5)
    return np.copysign(r, v)


def f16_bits_to_f64(bits):
    """Value of an IEEE binary16 bit pattern (finite patterns only), exactly."""
    b = np.asarray(bits, dtype=np.int64)
    sign = np.where(b & 0x8000, -1.0, 1.0)
    e = (b >> 10) & 0x1F
    m = (b & 0x3FF).astype(np.float64)
    if np.any(e == 0x1F):
        raise ValueError("inf/nan fp16 pattern")
    sub = m * 2.0 ** -24
    nrm = (1024.0 + m) * np.exp2(e.astype(np.float64) - 25.0)
    return sign * np.where(e == 0, sub, nrm)


def f16_ceil_div(v, c):
    """Smallest non-negative fp16 h with c*h >= v (v >= 0, c a small integer).

    Returns the fp16 bit pattern. c*h is exact in fp64 because h has at most 11
    significant bits and c at most 10. Saturates at the largest finite fp16
    (0x7BFF) if even that is too small. Binary search over the (monotone)
    bit patterns 0 .. 0x7BFF.
    """
    v = np.asarray(v, dtype=np.float64)
    lo = np.zeros(v.shape, dtype=np.int64)          # invariant: answer >= lo
    hi = np.full(v.shape, 0x7BFF, dtype=np.int64)   # invariant: answer <= hi
    for _ in range(16):
        mid = (lo + hi) // 2
        ok = c * f16_bits_to_f64(mid) >= v
        hi = np.where(ok, mid, hi)
        lo = np.where(ok, lo, mid + 1)
        lo = np.minimum(lo, hi)
    return hi


# --------------------------------------------------------------------------
# symmetric 32-blocks: Q8 activations, Q8_0 weights, Q4_0 weights
# --------------------------------------------------------------------------

def quantize_symmetric(x, qmax):
    """[P2] §5.1 applied to each 32-element block along the last axis.

    x: float32 array [..., K] with K % 32 == 0.
    Returns (q int64 [..., K], d float32 [..., K/32]):
      amax = max |x| over the block, d = amax / qmax (fp32 division),
      q = round_half_away(x / d) (fp32 division), clamped to [-qmax, qmax];
      d == 0 gives q == 0 (reading R5).
    """
    x = np.asarray(x, dtype=np.float32)
    K = x.shape[-1]
    if K % QK:
        raise ValueError("K must be a multiple of 32")
    xb = x.reshape(x.shape[:-1] + (K // QK, QK))
    amax = np.max(np.abs(xb), axis=-1)
    d = (amax / np.float32(qmax)).astype(np.float32)
    safe = np.where(d == 0, np.float32(1), d).astype(np.float32)
    v = (xb / safe[..., None]).astype(np.float32)      # fp32 IEEE division
    q = round_half_away(v.astype(np.float64))
    q = np.clip(q, -qmax, qmax)
    q = np.where((d == 0)[..., None], 0, q).astype(np.int64)
    return q.reshape(x.shape), d


def quantize_act(x):
    """Q8 activation blocks (reading R3): codes, scales and block sums.

    x: float32 [M, K]. Returns (q int64 [M,K], d float32 [M,K/32],
    s int64 [M,K/32]) with s = sum of the 32 codes of each block.
    """
    q, d = quantize_symmetric(x, 127)
    M, K = q.shape
    s = q.reshape(M, K // QK, QK).sum(axis=-1)
    return q, d, s


def quantize_q8_0(w):
    """[P2] §5.4 Q8_0: per 32-block int8 codes with an fp32 scale (b = 8)."""
    return quantize_symmetric(w, 127)


def quantize_q4_0(w):
    """[P2] §5.3 Q4_0 with the §5.1 rule at b = 4: q in [-7, 7], d = amax/7."""
    return quantize_symmetric(w, 7)


def fp16_round(x):
    """Nearest IEEE binary16 value of each fp32 number (ties to even), as
    float32; finite values beyond the fp16 range saturate at 65504 (R18)."""
    x = np.asarray(x, dtype=np.float32)
    with np.errstate(over="ignore"):
        h = x.astype(np.float16)
    h = np.where(np.isfinite(h), h, np.copysign(np.float16(65504), x))
    return h.astype(np.float32)


def quantize_q4_0_f16(w):
    """[P2] §5.3 Q4_0 as printed, with an fp16 scale (reading R18).

    w: float32 [..., K]. Returns (q int64 [..., K], d16 float32 [..., K/32]
    holding fp16 values): d16 = fp16(amax / 7), q = round_half_away(x / d16)
    in fp32, clamped to [-7, 7]; d16 == 0 gives q == 0.
    """
    x = np.asarray(w, dtype=np.float32)
    K = x.shape[-1]
    if K % QK:
        raise ValueError("K must be a multiple of 32")
    xb = x.reshape(x.shape[:-1] + (K // QK, QK))
    amax = np.max(np.abs(xb), axis=-1)
    d16 = fp16_round((amax / np.float32(7)).astype(np.float32))
    safe = np.where(d16 == 0, np.float32(1), d16).astype(np.float32)
    v = (xb / safe[..., None]).astype(np.float32)      # fp32 IEEE division
    q = np.clip(round_half_away(v.astype(np.float64)), -7, 7)
    q = np.where((d16 == 0)[..., None], 0, q).astype(np.int64)
    return q.reshape(x.shape), d16


def dequant_symmetric(q, d):
    """x^ = Q * scale ([P2] §5.1), per 32-block, in fp64."""
    q = np.asarray(q, dtype=np.float64)
    K = q.shape[-1]
    qb = q.reshape(q.shape[:-1] + (K // QK, QK))
    return (qb * np.asarray(d, np.float64)[..., None]).reshape(q.shape)


# --------------------------------------------------------------------------
# Q4_K super-blocks
# --------------------------------------------------------------------------

def quantize_q4_k(w):
    """Q4_K encoding of float32 rows w [N, K], K % 256 == 0.

    Per super-block of 256 ([P2] §5.5, [P4]) with sub-blocks j = 0..7 of 32,
    the asymmetric rule of [P2] §5.2 with the hierarchy of §5.5, in fp64:

      1. hi_j = max x, lo_j = min x over sub-block j.
      2. zero-point magnitude m_j = max(0, -lo_j)               (reading R7)
      3. dmin+ = smallest fp16 with 63*dmin+ >= max_j m_j         (reading R8)
      4. mn_j  = smallest integer in [0, 63] with mn_j*dmin+ >= m_j
         M_j   = mn_j * dmin+   (the zero point is -M_j <= lo_j)
      5. t_j   = hi_j + M_j     (the range the 16 levels must span)
      6. d     = smallest fp16 with 15*63*d >= max_j t_j          (reading R8)
      7. sc_j  = smallest integer in [0, 63] with 15*sc_j*d >= t_j
         S_j   = sc_j * d       (the sub-block scale, [P2] §5.5 scale_j)
      8. q_i   = clamp(round_half_away((x_i + M_j) / S_j), 0, 15), or 0 when
         S_j == 0   ([P2] §5.2 with zero_point = -M_j)
      9. stored d_min = -dmin+ so that x^ = (d*sc_j)*q + d_min*mn_j.

    Returns dict with d_bits, dmin_bits (uint16 [N, K/256]), sc, mn
    (int64 [N, K/256, 8]) and q (int64 [N, K], values 0..15).
    """
    w = np.asarray(w, dtype=np.float32)
    N, K = w.shape
    if K % QK_K:
        raise ValueError("K must be a multiple of 256")
    nsb = K // QK_K
    x = w.astype(np.float64).reshape(N, nsb, SUBS, QK)
    hi = x.max(axis=-1)
    lo = x.min(axis=-1)
    m = np.maximum(0.0, -lo)                                     # step 2
    dm_bits = f16_ceil_div(m.max(axis=-1), 63)                   # step 3
    dm = f16_bits_to_f64(dm_bits)
    k = np.arange(64, dtype=np.float64)
    mn = np.sum(k * dm[..., None, None] < m[..., None], axis=-1)  # step 4
    mn = np.minimum(mn, 63)
    Mj = mn * dm[..., None]
    t = hi + Mj                                                  # step 5
    d_bits = f16_ceil_div(t.max(axis=-1), 15 * 63)               # step 6
    d = f16_bits_to_f64(d_bits)
    sc = np.sum(15.0 * k * d[..., None, None] < t[..., None], axis=-1)  # 7
    sc = np.minimum(sc, 63)
    S = sc * d[..., None]
    safe = np.where(S == 0, 1.0, S)
    v = (x + Mj[..., None]) / safe[..., None]                    # step 8
    q = np.clip(round_half_away(v), 0, 15)
    q = np.where((S == 0)[..., None], 0, q).astype(np.int64)
    dmin_bits = np.where(dm_bits == 0, 0, dm_bits | 0x8000)      # step 9
    return dict(d_bits=d_bits.astype(np.uint16),
                dmin_bits=dmin_bits.astype(np.uint16),
                sc=sc.astype(np.int64), mn=mn.astype(np.int64),
                q=q.reshape(N, K))


def q4_k_sub_scales(enc):
    """Per-sub-block fp64 scale and min of [P2] §5.5:
    scale_j = d * scales[j], min_j = d_min * mins[j]. Shapes [N, K/32]."""
    d = f16_bits_to_f64(enc["d_bits"])
    dmin = f16_bits_to_f64(enc["dmin_bits"])
    scale = d[..., None] * enc["sc"]
    mins = dmin[..., None] * enc["mn"]
    N = scale.shape[0]
    return scale.reshape(N, -1), mins.reshape(N, -1)


def dequant_q4_k(enc):
    """[P2] §5.5: x^[32j + i] = qs[32j + i] * scale_j + min_j, fp64."""
    scale, mins = q4_k_sub_scales(enc)
    q = enc["q"].astype(np.float64)
    N, K = q.shape
    qb = q.reshape(N, K // QK, QK)
    return (qb * scale[..., None] + mins[..., None]).reshape(N, K)


# --------------------------------------------------------------------------
# packed byte layouts
# --------------------------------------------------------------------------

def _pad16(n):
    return (n + 15) // 16 * 16


def row_bytes(wtype, K):
    """Bytes of one packed weight row (header region, padded to 16 B, then
    the quant region)."""
    if wtype == TYPE_Q4_0:
        return _pad16(4 * (K // QK)) + 16 * (K // QK)
    if wtype == TYPE_Q8_0:
        return _pad16(4 * (K // QK)) + 32 * (K // QK)
    if wtype == TYPE_Q4_K:
        return 16 * (K // QK_K) + 128 * (K // QK_K)
    if wtype == TYPE_Q4_0_F16:
        return _pad16(2 * (K // QK)) + 16 * (K // QK)
    raise ValueError("unknown type")


def header_bytes(wtype, K):
    if wtype in (TYPE_Q4_0, TYPE_Q8_0):
        return _pad16(4 * (K // QK))
    if wtype == TYPE_Q4_0_F16:
        return _pad16(2 * (K // QK))
    return 16 * (K // QK_K)


def act_bytes(M, K):
    """Activation buffer: M*K int8 codes, then M*K/32 (fp32 d, int32 sum)."""
    return M * K + 8 * M * (K // QK)


def _nibble_pairs(codes):
    """Pack 4-bit codes (0..15) two per byte: byte t of a 32-block holds
    element 2t in the low nibble and 2t+1 in the high nibble ([P2] §6.4)."""
    c = np.asarray(codes, dtype=np.int64)
    lo = c[..., 0::2]
    hi = c[..., 1::2]
    return (lo | (hi << 4)).astype(np.uint8)


def _group8_permute(codes):
    """Reorder each group of 8 consecutive int8 codes to GROUP8_ORDER."""
    c = np.asarray(codes)
    sh = c.shape
    g = c.reshape(sh[:-1] + (sh[-1] // 8, 8))
    return g[..., GROUP8_ORDER].reshape(sh)


def _group8_unpermute(codes):
    c = np.asarray(codes)
    sh = c.shape
    g = c.reshape(sh[:-1] + (sh[-1] // 8, 8))
    out = np.empty_like(g)
    out[..., GROUP8_ORDER] = g
    return out.reshape(sh)


def pack_q4_0(q, d):
    """Rows of [fp32 d per block | pad to 16 B][16 B of nibbles per block],
    nibble = q + 8 (reading R2)."""
    q = np.asarray(q, dtype=np.int64)
    N, K = q.shape
    nb = K // QK
    out = np.zeros((N, row_bytes(TYPE_Q4_0, K)), dtype=np.uint8)
    out[:, :4 * nb] = np.asarray(d, dtype='<f4').reshape(N, nb).view(np.uint8)
    h = header_bytes(TYPE_Q4_0, K)
    out[:, h:] = _nibble_pairs(q + 8).reshape(N, 16 * nb)
    return out


def pack_q4_0_f16(q, d16):
    """Rows of [fp16 d per block | pad to 16 B][16 B of nibbles per block],
    nibble = q + 8: [P2] §5.3's 18 bytes per 32 weights, split by row into a
    scale region and a code region like the other types."""
    q = np.asarray(q, dtype=np.int64)
    N, K = q.shape
    nb = K // QK
    out = np.zeros((N, row_bytes(TYPE_Q4_0_F16, K)), dtype=np.uint8)
    out[:, :2 * nb] = np.asarray(d16, dtype='<f2').reshape(N, nb).view(np.uint8)
    h = header_bytes(TYPE_Q4_0_F16, K)
    out[:, h:] = _nibble_pairs(q + 8).reshape(N, 16 * nb)
    return out


def pack_q8_0(q, d):
    """Rows of [fp32 d per block | pad to 16 B][32 int8 per block, each group
    of 8 in GROUP8_ORDER]."""
    q = np.asarray(q, dtype=np.int64)
    N, K = q.shape
    nb = K // QK
    out = np.zeros((N, row_bytes(TYPE_Q8_0, K)), dtype=np.uint8)
    out[:, :4 * nb] = np.asarray(d, dtype='<f4').reshape(N, nb).view(np.uint8)
    h = header_bytes(TYPE_Q8_0, K)
    out[:, h:] = _group8_permute(q).astype(np.int8).view(np.uint8)
    return out


def pack_q4_k(enc):
    """Rows of [16 B header per super-block][128 B of nibbles per super-block].

    Header: d (fp16), d_min (fp16), then a 96-bit little-endian field with
    sc_j at bits [6j, 6j+6) and mn_j at bits [48+6j, 48+6j+6), j = 0..7.
    Nibbles: sub-block j of a super-block is bytes [16j, 16j+16) of its 128,
    byte t holding element 32j+2t (low) and 32j+2t+1 (high).
    """
    q = enc["q"]
    N, K = q.shape
    nsb = K // QK_K
    hdr = np.zeros((N, nsb, 16), dtype=np.uint8)
    hdr[..., 0:2] = enc["d_bits"].astype('<u2')[..., None].view(np.uint8)
    hdr[..., 2:4] = enc["dmin_bits"].astype('<u2')[..., None].view(np.uint8)
    field = np.zeros((N, nsb), dtype=object)
    for j in range(SUBS):
        field = field + (enc["sc"][..., j].astype(object) << (6 * j))
        field = field + (enc["mn"][..., j].astype(object) << (48 + 6 * j))
    for byte in range(12):
        hdr[..., 4 + byte] = ((field >> (8 * byte)) & 0xFF).astype(np.uint8)
    out = np.zeros((N, row_bytes(TYPE_Q4_K, K)), dtype=np.uint8)
    out[:, :16 * nsb] = hdr.reshape(N, 16 * nsb)
    out[:, 16 * nsb:] = _nibble_pairs(q).reshape(N, 128 * nsb)
    return out


def unpack_q4_k(packed, K):
    """Inverse of pack_q4_k (used to read device-packed buffers back)."""
    packed = np.asarray(packed, dtype=np.uint8)
    N = packed.shape[0]
    nsb = K // QK_K
    hdr = packed[:, :16 * nsb].reshape(N, nsb, 16)
    d_bits = hdr[..., 0:2].copy().view('<u2')[..., 0]
    dmin_bits = hdr[..., 2:4].copy().view('<u2')[..., 0]
    field = np.zeros((N, nsb), dtype=object)
    for byte in range(12):
        field = field + (hdr[..., 4 + byte].astype(object) << (8 * byte))
    sc = np.zeros((N, nsb, SUBS), dtype=np.int64)
    mn = np.zeros((N, nsb, SUBS), dtype=np.int64)
    for j in range(SUBS):
        sc[..., j] = ((field >> (6 * j)) & 63).astype(np.int64)
        mn[..., j] = ((field >> (48 + 6 * j)) & 63).astype(np.int64)
    nib = packed[:, 16 * nsb:].astype(np.int64)
    q = np.empty((N, K), dtype=np.int64)
    q[:, 0::2] = nib & 15
    q[:, 1::2] = nib >> 4
    return dict(d_bits=d_bits, dmin_bits=dmin_bits, sc=sc, mn=mn, q=q)


def unpack_q4_0(packed, K):
    packed = np.asarray(packed, dtype=np.uint8)
    N = packed.shape[0]
    nb = K // QK
    d = packed[:, :4 * nb].copy().view('<f4').reshape(N, nb)
    nib = packed[:, header_bytes(TYPE_Q4_0, K):].astype(np.int64)
    q = np.empty((N, K), dtype=np.int64)
    q[:, 0::2] = (nib & 15) - 8
    q[:, 1::2] = (nib >> 4) - 8
    return q, d


def unpack_q4_0_f16(packed, K):
    packed = np.asarray(packed, dtype=np.uint8)
    N = packed.shape[0]
    nb = K // QK
    d16 = packed[:, :2 * nb].copy().view('<f2').reshape(N, nb).astype(np.float32)
    nib = packed[:, header_bytes(TYPE_Q4_0_F16, K):].astype(np.int64)
    q = np.empty((N, K), dtype=np.int64)
    q[:, 0::2] = (nib & 15) - 8
    q[:, 1::2] = (nib >> 4) - 8
    return q, d16


def unpack_q8_0(packed, K):
    packed = np.asarray(packed, dtype=np.uint8)
    N = packed.shape[0]
    nb = K // QK
    d = packed[:, :4 * nb].copy().view('<f4').reshape(N, nb)
    raw = packed[:, header_bytes(TYPE_Q8_0, K):].copy().view(np.int8)
    q = _group8_unpermute(raw.astype(np.int64))
    return q, d


def pack_act(q, d, s):
    """Activation buffer bytes: [M*K int8 codes, each group of 8 in
    GROUP8_ORDER][M*K/32 pairs of (fp32 d, int32 sum)], row-major in m."""
    q = np.asarray(q, dtype=np.int64)
    M, K = q.shape
    nb = K // QK
    codes = _group8_permute(q).astype(np.int8).view(np.uint8).reshape(-1)
    ds = np.zeros((M, nb, 2), dtype='<u4')
    ds[..., 0] = np.asarray(d, dtype='<f4').view('<u4')
    ds[..., 1] = np.asarray(s, dtype=np.int64).astype('<i4').view('<u4')
    return np.concatenate([codes, ds.view(np.uint8).reshape(-1)])


def unpack_act(buf, M, K):
    buf = np.asarray(buf, dtype=np.uint8)
    nb = K // QK
    codes = buf[:M * K].copy().view(np.int8).reshape(M, K).astype(np.int64)
    ds = buf[M * K:M * K + 8 * M * nb].copy().view('<u4').reshape(M, nb, 2)
    d = ds[..., 0].copy().view('<f4')
    s = ds[..., 1].copy().view('<i4').astype(np.int64)
    return _group8_unpermute(codes), d, s


# --------------------------------------------------------------------------
# the quantized product
# --------------------------------------------------------------------------

def block_sums(wq, aq):
    """Integer block dot products S[m, n, b] = sum_i wq[n, 32b+i]*aq[m, 32b+i]
    in int64 ([P3] §2.2: integer multiply-add inside each block).

    wq: int [N, K] weight codes (Q4_0: q = nibble - 8; Q8_0: q;
    Q4_K: the raw nibble 0..15). aq: int [M, K] activation codes.
    """
    wq = np.asarray(wq, dtype=np.int64)
    aq = np.asarray(aq, dtype=np.int64)
    N, K = wq.shape
    M = aq.shape[0]
    nb = K // QK
    return np.einsum("mbi,nbi->mnb", aq.reshape(M, nb, QK),
                     wq.reshape(N, nb, QK), dtype=np.int64)


def product_sym(wq, dw, aq, da):
    """Q4_0 / Q8_0 product: y[m, n] = sum_b dw[n,b]*da[m,b]*S[m,n,b].

    The scales are applied outside the integer block dot ([P2] §6.4 applies d
    per block; [P3] §2.2). Evaluated in fp64, rounded once to fp32.
    Returns (y32, y64), shape [M, N].
    """
    S = block_sums(wq, aq).astype(np.float64)
    y = np.einsum("mnb,nb,mb->mn", S, np.asarray(dw, np.float64),
                  np.asarray(da, np.float64))
    return y.astype(np.float32), y


def product_q4_k(enc, aq, da, sa):
    """Q4_K product, with activation block b aligned to sub-block b % 8 of
    super-block b // 8:

      y[m, n] = sum_b da[m,b] * ( scale[n,b] * S[m,n,b] + min[n,b] * A[m,b] )

    where scale/min are [P2] §5.5's scale_j and min_j, S is the integer dot of
    the raw nibbles with the activation codes and A[m, b] = sum of the
    activation codes of block b. This is sum_i da*aq_i*(scale*q_i + min),
    i.e. [P2] §5.5's dequantized weight times the dequantized activation,
    regrouped so the only per-element work is integer. fp64, rounded once.
    """
    scale, mins = q4_k_sub_scales(enc)
    S = block_sums(enc["q"], aq).astype(np.float64)
    A = np.asarray(sa, np.float64)
    da = np.asarray(da, np.float64)
    y = (np.einsum("mnb,nb,mb->mn", S, scale, da)
         + np.einsum("mb,nb,mb->mn", A, mins, da))
    return y.astype(np.float32), y


def dequant_dot(wdeq, adeq):
    """fp64 dot product of the dequantized operands: Y = adeq @ wdeq^T."""
    return np.asarray(adeq, np.float64) @ np.asarray(wdeq, np.float64).T


def product_float(wtype, enc, x):
    """Float-activation product (R12): [P2] §6.4's scalar Q4_0 kernel decodes
    each weight in place, (nibble - 8) * d, and multiplies it by a float
    activation; the other formats decode as their dequantization rule
    ([P2] §5.4 Q8_0, §5.5 Q4_K). y[m, n] = sum_k w^[n, k] * x[m, k] with w^
    the dequantized weights, in fp64 from the given x, rounded once.
    Returns (y32, y64), shape [M, N]."""
    y = dequant_dot(dequant_weights(wtype, enc), np.asarray(x, np.float64))
    return y.astype(np.float32), y


# --------------------------------------------------------------------------
# whole-path helpers: float inputs -> quantize -> product
# --------------------------------------------------------------------------

def encode_weights(wtype, w):
    """Quantize and pack float32 weights. Returns (packed uint8 [N, rb], enc)
    where enc holds the codes and scales."""
    if wtype == TYPE_Q4_0:
        q, d = quantize_q4_0(w)
        return pack_q4_0(q, d), dict(q=q, d=d)
    if wtype == TYPE_Q8_0:
        q, d = quantize_q8_0(w)
        return pack_q8_0(q, d), dict(q=q, d=d)
    if wtype == TYPE_Q4_K:
        enc = quantize_q4_k(w)
        return pack_q4_k(enc), enc
    if wtype == TYPE_Q4_0_F16:
        q, d = quantize_q4_0_f16(w)
        return pack_q4_0_f16(q, d), dict(q=q, d=d)
    raise ValueError("unknown type")


def product(wtype, enc, act):
    """y32, y64 [M, N] for encoded weights and (q, d, s) activations."""
    aq, da, sa = act
    if wtype in (TYPE_Q4_0, TYPE_Q8_0, TYPE_Q4_0_F16):
        return product_sym(enc["q"], enc["d"], aq, da)
    return product_q4_k(enc, aq, da, sa)


def weight_codes_for_sums(wtype, enc):
    """The integer weight codes whose block dot with the activation codes is
    the integer block sum of each format (Q4_0: nibble-8, Q8_0: q,
    Q4_K: raw nibble)."""
    return enc["q"]


def dequant_weights(wtype, enc):
    if wtype in (TYPE_Q4_0, TYPE_Q8_0, TYPE_Q4_0_F16):
        return dequant_symmetric(enc["q"], enc["d"])
    return dequant_q4_k(enc)


# --------------------------------------------------------------------------
# quantized KV cache ([P2] §3.7.1 K/V of earlier tokens are kept; §3.7.3 the
# cache may be stored as Q8_0 or Q4_0)
# --------------------------------------------------------------------------

def kv_scores(wtype, k, q, n_head):
    """Scores of n_head queries against a quantized K cache.

    k: fp32 [n_kv, n_tok, head_dim], the keys of every cached token, each
    token's head_dim values quantized like one weight row of type wtype.
    q: fp32 [n_head, head_dim], quantized like activations (R3).
    Query head hq reads KV head h = hq // (n_head // n_kv) (grouped queries).
    scores[hq, t] is the weight-product of key row (h, t) with query hq.
    Returns (y32, y64), shape [n_head, n_tok]."""
    k = np.asarray(k, np.float32)
    n_kv, n_tok, _ = k.shape
    group = n_head // n_kv
    aq, da, sa = quantize_act(q)
    y = np.zeros((n_head, n_tok), np.float64)
    for hq in range(n_head):
        _, enc = encode_weights(wtype, k[hq // group])
        y[hq] = product(wtype, enc, (aq[hq:hq + 1], da[hq:hq + 1], sa[hq:hq + 1]))[1][0]
    return y.astype(np.float32), y


def rel_err(y, yref):
    """max |y - yref| / max |yref| over the whole output (0 if both are 0)."""
    y = np.asarray(y, np.float64)
    yref = np.asarray(yref, np.float64)
    den = np.max(np.abs(yref)) if yref.size else 0.0
    num = np.max(np.abs(y - yref)) if yref.size else 0.0
    if den == 0.0:
        return 0.0 if num == 0.0 else np.inf
    return num / den
