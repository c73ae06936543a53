// Prefill-path product Y[m][n] = X * W^T for few activation rows (m <= 64).
//
// With few rows the 128 x 128 tiles of the main GEMM leave most of the chip
// idle and most of each tile empty, while the product is still a stream of
// the whole weight matrix. This form keeps every weight byte read once and
// spreads the work over many small workgroups instead:
//   * a workgroup owns 16 * NT weight rows (columns n of Y: 64, or 32 and
//     16 for short matrices, so the grid fills the chip) and all m rows of X,
//     padded to 16 * MT;
//   * its four waves split the reduction over k into four contiguous,
//     super-block-aligned quarters and add their partial tiles in LDS at the
//     end, in a fixed order (the result does not depend on scheduling);
//   * each 32-block's integer dot product is one v_mfma_i32_16x16x32_i8 over
//     a 16 x 16 tile (K = 32 is exactly one block; "llama.cpp 推理引擎", §6.4:
//     the scales stay outside the integer values), its scales are applied in
//     fp32 right after it (Q4_K: §5.5, d*sc_j and d_min*mn_j), and the
//     per-block min terms run on the matrix cores as an fp32 product over
//     blocks (v_mfma_f32_16x16x4f32, four blocks per instruction).
//
// Tiles are computed transposed, D[n][m]: the weights are the A operand, so
// each lane holds one activation row (one activation scale per block) and
// four consecutive weight rows (one float4 of weight scales per block).
// Operands come straight from global memory into registers as whole blocks
// (16-byte loads), one 4-block group ahead of the compute, and are exchanged
// across lanes into the MFMA operand layout with permlane swaps; the weight
// scales of the next super-block (8 blocks) are loaded one super-block ahead
// and decoded into a small wave-private LDS table.
//
// Operand pairing: lane group q = lane / 16 of a 16x16x32 MFMA holds block
// elements [8q, 8q + 8). The activation codes of a block are stored in the
// order 0,2,4,6,1,3,5,7 within groups of 8, and the 4-bit weights of a
// block, unpacked as (low nibbles, high nibbles) of bytes [4q, 4q + 4),
// yield the same element order, so both operands pair up element by element.
#include "qblk_device.h"

namespace qblk {
namespace {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((__vector_size__(2 * sizeof(unsigned int))));

constexpr int kSb = 8;  // blocks per scale chunk (one Q4_K super-block)
// waves per workgroup = ways the k range is split (measured on MI355X: 8 or
// 16 waves, or loads a whole chunk ahead, are slower for 1..64 rows)
constexpr int kWaves = 4;
// kMagicBits / kMagic (fp32 1.5 * 2^23): qblk_device.h

template <int TYPE>
constexpr bool kHasMin = TYPE != kQ8_0;

// Wave-private table of decoded weight scales for one 8-block chunk of the
// workgroup's 16 * NT weight rows: sw = block scale (Q4_K: d * sc_j), wm = min
// coefficient (Q4_K: d_min * mn_j; Q4_0: -8 d). Blocks past the wave's range
// hold zeros.
template <int NT>
struct ScaleTable {
  float sw[kSb][16 * NT];
  float wm[kSb][16 * NT];
};

// LDS of a workgroup: the waves' scale tables during the loop, then their
// partial tiles for the final sum.
template <int MT, int NT, int WAVES>
union Shared {
  ScaleTable<NT> tab[WAVES];
  float red[WAVES][MT][NT][4][64];
};

// The table of a chunk is filled by all 64 lanes: lane = (column c, part h)
// with c = lane % (16 NT) and P = 64 / (16 NT) parts per column. Raw data of
// one lane: Q4_K = the column's super-block header (part h decodes values
// [16h/P, 16(h+1)/P) of its 8 scale and 8 min codes); other types = the block
// scales (fp32, or fp16 for Q4_0_F16) of blocks [c0 + h 8/P, c0 + (h+1) 8/P).
struct RawScales {
  uint4 v[2];
};

template <int NT>
constexpr int kParts = 64 / (16 * NT);

template <int TYPE, int NT>
__device__ __forceinline__ RawScales load_scales(const WeightView& W, int64_t n0, int64_t n, int64_t nb,
                                                 int64_t c0, int lane) {
  constexpr int P = kParts<NT>;
  constexpr int kBlk = kSb / P;  // blocks per part (non-K types)
  RawScales r;
  r.v[0] = r.v[1] = make_uint4(0, 0, 0, 0);
  const int col = lane % (16 * NT);
  const int h = lane / (16 * NT);
  const int64_t gn = n0 + col < n ? n0 + col : n - 1;
  const uint8_t* row = W.row(gn);
  if constexpr (TYPE == kQ4_K) {
    r.v[0] = load16(row + 16 * (c0 / kSb));
  } else {
    const int64_t b = c0 + kBlk * h;
    // reads stay inside the zero-padded header: b and b + 4 are multiples of
    // 4 blocks, each read only when its first block exists
    if constexpr (TYPE == kQ4_0H) {
      if (b < nb) {
        if constexpr (kBlk == 8) r.v[0] = load16(row + 2 * b);
        else if constexpr (kBlk == 4) { const uint2 x = *reinterpret_cast<const uint2*>(row + 2 * b); r.v[0] = make_uint4(x.x, x.y, 0, 0); }
        else r.v[0].x = *reinterpret_cast<const uint32_t*>(row + 2 * b);
      }
    } else {
      if (b < nb) {
        if constexpr (kBlk >= 4) r.v[0] = load16(row + 4 * b);
        else { const uint2 x = *reinterpret_cast<const uint2*>(row + 4 * b); r.v[0] = make_uint4(x.x, x.y, 0, 0); }
      }
      if constexpr (kBlk == 8) {
        if (b + 4 < nb) r.v[1] = load16(row + 4 * (b + 4));
      }
    }
  }
  return r;
}

// Bits [b, b + 6) of the Q4_K header's 96-bit scale/min field (h.y = bits
// 0..31, h.z = 32..63, h.w = 64..95); b is a compile-time constant after
// unrolling, so this is one funnel shift and a mask.
__device__ __forceinline__ uint32_t field6(const uint4& h, int b) {
  const uint32_t lo = b < 32 ? h.y : b < 64 ? h.z : h.w;
  const uint32_t hi = b < 32 ? h.z : b < 64 ? h.w : 0u;
  return __builtin_amdgcn_alignbit(hi, lo, b & 31) & 63u;
}

// Decode one chunk into the table; blocks at or past `jend` get zeros.
template <int TYPE, int NT>
__device__ __forceinline__ void decode_scales(ScaleTable<NT>* __restrict__ t, const RawScales& r, int64_t c0,
                                              int64_t jend, int lane) {
  constexpr int P = kParts<NT>;
  const int col = lane % (16 * NT);
  const int h = lane / (16 * NT);
  if constexpr (TYPE == kQ4_K) {
    // jend is a multiple of 8 here (k is a multiple of 256): the chunk is whole
    constexpr int kVals = 16 / P;
    const float d = half_bits_to_float(r.v[0].x);
    const float dmin = half_bits_to_float(r.v[0].x >> 16);
#pragma unroll
    for (int pp = 0; pp < P; ++pp) {
      if (h == pp) {  // the part index is a compile-time constant inside
#pragma unroll
        for (int i = 0; i < kVals; ++i) {
          const int v = pp * kVals + i;
          if (v < 8) t->sw[v][col] = d * static_cast<float>(field6(r.v[0], 6 * v));              // sc_v
          else t->wm[v - 8][col] = dmin * static_cast<float>(field6(r.v[0], 48 + 6 * (v - 8)));  // mn_(v-8)
        }
      }
    }
  } else {
    constexpr int kBlk = kSb / P;
    float d[kBlk];
#pragma unroll
    for (int i = 0; i < kBlk; ++i) {
      if constexpr (TYPE == kQ4_0H) {
        const uint32_t w = i < 2 ? r.v[0].x : i < 4 ? r.v[0].y : i < 6 ? r.v[0].z : r.v[0].w;
        d[i] = half_bits_to_float(w >> (16 * (i & 1)));
      } else {
        const uint4& v = r.v[i / 4];
        const int e = i % 4;
        d[i] = __uint_as_float(e == 0 ? v.x : e == 1 ? v.y : e == 2 ? v.z : v.w);
      }
    }
#pragma unroll
    for (int i = 0; i < kBlk; ++i) {
      const bool ok = c0 + kBlk * h + i < jend;
      t->sw[kBlk * h + i][col] = ok ? d[i] : 0.0f;
      if constexpr (kHasMin<TYPE>) t->wm[kBlk * h + i][col] = ok ? -8.0f * d[i] : 0.0f;  // nibble - 8
    }
  }
}

// Operands of one 4-block group as loaded: lane (r, q) = (lane % 16,
// lane / 16) reads whole blocks, block j0 + q of its weight / activation row,
// with 16-byte loads (each load instruction covers 64 or 128 contiguous bytes
// of 16 rows). A 4 x 4 exchange across the four 16-lane rows then hands each
// lane the element group q of every block of the group, the operand layout of
// the 16x16x32 MFMA.
template <int TYPE, int MT, int NT>
struct Ops {
  static constexpr int kWDwords = TYPE == kQ8_0 ? 8 : 4;
  uint32_t w[NT][kWDwords];  // block j0 + q of weight row 16 nt + r
  uint32_t a[MT][8];         // block j0 + q of activation row 16 mt + r
  float2 own[MT];            // (d, code sum) of that activation block
};

// 4 x 4 transpose across the four 16-lane rows of the wave: on entry lane
// (c, q) holds x[0..3]; on exit x[i] of lane (c, q) is the entry x[q] of lane
// (c, i). Two 32-lane and two 16-lane swaps (gfx950 permlane swaps).
__device__ __forceinline__ void transpose4(uint32_t& x0, uint32_t& x1, uint32_t& x2, uint32_t& x3) {
  auto p = __builtin_amdgcn_permlane32_swap(x0, x2, false, false);
  x0 = p[0];
  x2 = p[1];
  p = __builtin_amdgcn_permlane32_swap(x1, x3, false, false);
  x1 = p[0];
  x3 = p[1];
  p = __builtin_amdgcn_permlane16_swap(x0, x1, false, false);
  x0 = p[0];
  x1 = p[1];
  p = __builtin_amdgcn_permlane16_swap(x2, x3, false, false);
  x2 = p[0];
  x3 = p[1];
}

// Buffer views of the operands. Raw buffer loads return zeros past
// `num_records` instead of faulting, and take a wave-uniform base plus a
// 32-bit per-lane offset, so a group's loads share one offset register and
// differ only in their immediate offsets.
struct Sources {
  __amdgpu_buffer_rsrc_t w;    // this workgroup's weight rows
  __amdgpu_buffer_rsrc_t a;    // activation codes [m][k]
  __amdgpu_buffer_rsrc_t ds;   // activation (d, code sum) pairs [m][nb]
  uint32_t w_off[4];           // byte offset of block q of weight row 16 nt + r
  uint32_t a_off[4];           // byte offset of block q of activation row 16 mt + r
  uint32_t ds_off[4];          // byte offset of block q's pair of activation row 16 mt + r
};

constexpr int kBufferWord3 = 0x00020000;  // raw 32-bit buffer, range-checked

// Loads of the group of 4 blocks starting at j0. Weight rows past n and
// activation rows past m lie past their buffers and read as zeros; blocks
// past the wave's range are read (they lie inside the buffers or past them)
// and their contribution is cancelled by a zero activation scale.
template <int TYPE, int MT, int NT>
__device__ __forceinline__ void load_ops(Ops<TYPE, MT, NT>& o, const Sources& src, int64_t j0) {
  constexpr uint32_t kWBlk = TYPE == kQ8_0 ? 32u : 16u;
  const uint32_t jw = static_cast<uint32_t>(j0) * kWBlk;
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
#pragma unroll
    for (int h = 0; h < Ops<TYPE, MT, NT>::kWDwords / 4; ++h) {
      const auto v = __builtin_amdgcn_raw_buffer_load_b128(src.w, src.w_off[nt] + jw + 16 * h, 0, 0);
#pragma unroll
      for (int i = 0; i < 4; ++i) o.w[nt][4 * h + i] = v[i];
    }
  }
  const uint32_t ja = static_cast<uint32_t>(j0) * 32u, jd = static_cast<uint32_t>(j0) * 8u;
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) {
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const auto v = __builtin_amdgcn_raw_buffer_load_b128(src.a, src.a_off[mt] + ja + 16 * h, 0, 0);
#pragma unroll
      for (int i = 0; i < 4; ++i) o.a[mt][4 * h + i] = v[i];
    }
    const u32x2 p = __builtin_amdgcn_raw_buffer_load_b64(src.ds, src.ds_off[mt] + jd, 0, 0);
    o.own[mt] = make_float2(__uint_as_float(p[0]), __uint_as_float(p[1]));
  }
}

__device__ __forceinline__ long pack64(uint32_t lo, uint32_t hi) {
  return static_cast<long>(static_cast<uint64_t>(lo) | (static_cast<uint64_t>(hi) << 32));
}

template <int TYPE, int MT, int NT>
__device__ __forceinline__ void compute_group(Ops<TYPE, MT, NT> o, const ScaleTable<NT>* __restrict__ t, int jt,
                                              int64_t j0, int64_t jend, int q, int r, v4f (&acc)[MT][NT]) {
  // exchange: afterwards the 4-bit weights' w[nt][jj], the 8-bit weights'
  // (w[nt][2 jj], w[nt][2 jj + 1]) and the activations' (a[mt][2 jj],
  // a[mt][2 jj + 1]) are element group q of block j0 + jj, and d[mt][jj] is
  // the activation scale of block j0 + jj
  uint32_t d[MT][4];
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
    if constexpr (TYPE == kQ8_0) {
      transpose4(o.w[nt][0], o.w[nt][2], o.w[nt][4], o.w[nt][6]);
      transpose4(o.w[nt][1], o.w[nt][3], o.w[nt][5], o.w[nt][7]);
    } else {
      transpose4(o.w[nt][0], o.w[nt][1], o.w[nt][2], o.w[nt][3]);
    }
  }
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) {
    transpose4(o.a[mt][0], o.a[mt][2], o.a[mt][4], o.a[mt][6]);
    transpose4(o.a[mt][1], o.a[mt][3], o.a[mt][5], o.a[mt][7]);
#pragma unroll
    for (int i = 0; i < 4; ++i) d[mt][i] = __float_as_uint(o.own[mt].x);
    transpose4(d[mt][0], d[mt][1], d[mt][2], d[mt][3]);
  }

  v4i cinit;
#pragma unroll
  for (int v = 0; v < 4; ++v) cinit[v] = TYPE == kQ4_K ? kMagicBits : 0;
#pragma unroll
  for (int jj = 0; jj < 4; ++jj) {
    const bool ok = j0 + jj < jend;  // wave-uniform
    v4f sw[NT], ncs[NT];
    long wop[NT];
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      sw[nt] = *reinterpret_cast<const v4f*>(&t->sw[jt + jj][16 * nt + 4 * q]);
      ncs[nt] = -kMagic * sw[nt];
      if constexpr (TYPE == kQ8_0) {
        wop[nt] = pack64(o.w[nt][2 * jj], o.w[nt][2 * jj + 1]);
      } else {
        const uint32_t msk = 0x0F0F0F0Fu, w = o.w[nt][jj];
        wop[nt] = pack64(w & msk, (w >> 4) & msk);  // low nibbles, then high nibbles
      }
    }
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      const float sa = ok ? __uint_as_float(d[mt][jj]) : 0.0f;
      const long aop = pack64(o.a[mt][2 * jj], o.a[mt][2 * jj + 1]);
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) {
        const v4i c = __builtin_amdgcn_mfma_i32_16x16x32_i8(wop[nt], aop, cinit, 0, 0, 0);
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          float s;
          if constexpr (TYPE == kQ4_K)
            s = fmaf(__int_as_float(c[v]), sw[nt][v], ncs[nt][v]);  // = round(S * sw), exact S
          else
            s = static_cast<float>(c[v]) * sw[nt][v];
          acc[mt][nt][v] = fmaf(s, sa, acc[mt][nt][v]);
        }
      }
    }
    __builtin_amdgcn_sched_barrier(0);  // one block's MFMA results live at a time
  }
  if constexpr (kHasMin<TYPE>) {
    // min terms of the 4 blocks: A[n][b] = wm, B[b][m] = d * code sum
    const bool okq = j0 + q < jend;
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      const float asc = okq ? o.own[mt].x * static_cast<float>(__float_as_int(o.own[mt].y)) : 0.0f;
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) {
        const float wm = t->wm[jt + q][16 * nt + r];
        acc[mt][nt] = __builtin_amdgcn_mfma_f32_16x16x4f32(wm, asc, acc[mt][nt], 0, 0, 0);
      }
    }
  }
}

template <int TYPE, int MT, int NT, int WAVES, bool CHUNKS>
__global__ __launch_bounds__(64 * WAVES) void gemm_small_kernel(WeightView W, int64_t n, int64_t nb, ActView A,
                                                                int64_t m, float* __restrict__ y, int64_t ldy) {
  static_assert(MT <= 4 && NT <= 4, "operand offsets are sized for 4 x 4 tiles");
  __shared__ __attribute__((aligned(16))) Shared<MT, NT, WAVES> sh;
  // CHUNKS (more than 64 rows): blockIdx.y picks this workgroup's 16 MT
  // activation rows (a separate instance: the offsets cost the 64-row
  // instance, at its register limit, 7% at 14336 x 4096)
  if constexpr (CHUNKS) {
    const int64_t m0 = static_cast<int64_t>(blockIdx.y) * (16 * MT);
    A.q += m0 * A.k;
    A.ds += m0 * nb * 8;
    y += m0 * ldy;
    m = m - m0 < 16 * MT ? m - m0 : 16 * MT;
  }
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int q = lane >> 4;   // element group of the block / weight-row quad of the tile
  const int r = lane & 15;   // weight row (A operand) / activation row (B operand, D column)
  const int64_t n0 = static_cast<int64_t>(blockIdx.x) * (16 * NT);

  // this wave's blocks: a quarter of the row, aligned to whole chunks
  const int64_t per = (((nb + WAVES - 1) / WAVES) + kSb - 1) / kSb * kSb;
  const int64_t jbeg = per * wave < nb ? per * wave : nb;
  const int64_t jend = per * (wave + 1) < nb ? per * (wave + 1) : nb;

  v4f acc[MT][NT];
#pragma unroll
  for (int a = 0; a < MT; ++a)
#pragma unroll
    for (int b = 0; b < NT; ++b) acc[a][b] = v4f{0.0f, 0.0f, 0.0f, 0.0f};

  if (jbeg < jend) {
    Sources src;
    const int64_t rows = n - n0 < 16 * NT ? n - n0 : 16 * NT;
    src.w = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(W.row(n0)), 0,
                                              static_cast<int>(rows * W.row_bytes), kBufferWord3);
    src.a = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(A.q), 0, static_cast<int>(m * A.k),
                                              kBufferWord3);
    src.ds = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(A.ds), 0, static_cast<int>(m * nb * 8),
                                               kBufferWord3);
#pragma unroll
    for (int nt = 0; nt < NT; ++nt)
      src.w_off[nt] = static_cast<uint32_t>((16 * nt + r) * W.row_bytes + W.hdr_bytes) +
                      (TYPE == kQ8_0 ? 32u : 16u) * q;
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      src.a_off[mt] = static_cast<uint32_t>((16 * mt + r) * A.k) + 32u * q;
      src.ds_off[mt] = static_cast<uint32_t>((16 * mt + r) * nb * 8) + 8u * q;
    }
    ScaleTable<NT>* tab = &sh.tab[wave];

    // two operand sets in turn: group 0 of a chunk computes from `ga` while
    // group 1's operands stream into `gb`, then the roles swap (no register
    // copies, so a load is only waited for where its data is used)
    Ops<TYPE, MT, NT> ga, gb;
    const RawScales raw0 = load_scales<TYPE, NT>(W, n0, n, nb, jbeg, lane);
    load_ops<TYPE, MT, NT>(ga, src, jbeg);  // in flight while the first table is decoded
    decode_scales<TYPE, NT>(tab, raw0, jbeg, jend, lane);
    for (int64_t c0 = jbeg; c0 < jend; c0 += kSb) {
      const bool more = c0 + kSb < jend;  // wave-uniform
      const bool second = c0 + 4 < jend;
      // the loads are issued on every path, so the wait before each use
      // counts only the loads issued after it
      const RawScales raw = load_scales<TYPE, NT>(W, n0, n, nb, more ? c0 + kSb : c0, lane);
      load_ops<TYPE, MT, NT>(gb, src, c0 + 4);
      asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");  // the table of chunk c0 is written
      compute_group<TYPE, MT, NT>(ga, tab, 0, c0, jend, q, r, acc);
      load_ops<TYPE, MT, NT>(ga, src, c0 + kSb);
      if (second) compute_group<TYPE, MT, NT>(gb, tab, 4, c0 + 4, jend, q, r, acc);
      asm volatile("" ::: "memory");  // table reads of this chunk stay before its rewrite
      if (more) decode_scales<TYPE, NT>(tab, raw, c0 + kSb, jend, lane);
    }
  }

  // ---- partial tiles of the waves' k ranges, summed in wave order
  __syncthreads();  // all scale tables are done with (they share the LDS)
#pragma unroll
  for (int a = 0; a < MT; ++a)
#pragma unroll
    for (int b = 0; b < NT; ++b)
#pragma unroll
      for (int v = 0; v < 4; ++v) sh.red[wave][a][b][v][lane] = acc[a][b][v];
  __syncthreads();
  constexpr int kOut = 16 * MT * 16 * NT;
  for (int e = tid; e < kOut; e += 64 * WAVES) {
    const int mm = e / (16 * NT);
    const int nn = e % (16 * NT);
    const int64_t gm = mm, gn = n0 + nn;
    if (gm >= m || gn >= n) continue;
    const int mt = mm >> 4, c = mm & 15;
    const int nt = nn >> 4, v = nn & 3, qq = (nn & 15) >> 2;
    const int ln = 16 * qq + c;
    float s = sh.red[0][mt][nt][v][ln];
#pragma unroll
    for (int w = 1; w < WAVES; ++w) s += sh.red[w][mt][nt][v][ln];
    y[gm * ldy + gn] = s;
  }
}

template <int TYPE, int MT, int NT, int WAVES>
void launch_t(const WeightView& W, int64_t n, int64_t nb, const ActView& A, int64_t m, float* y, int64_t ldy,
              hipStream_t s) {
  const dim3 grid(static_cast<uint32_t>((n + 16 * NT - 1) / (16 * NT)),
                  static_cast<uint32_t>((m + 16 * MT - 1) / (16 * MT)));
  if (m > 16 * MT)
    hipLaunchKernelGGL((gemm_small_kernel<TYPE, MT, NT, WAVES, true>), grid, dim3(64 * WAVES), 0, s, W, n, nb, A, m,
                       y, ldy);
  else
    hipLaunchKernelGGL((gemm_small_kernel<TYPE, MT, NT, WAVES, false>), grid, dim3(64 * WAVES), 0, s, W, n, nb, A,
                       m, y, ldy);
}

template <int TYPE, int NT>
void launch_nt(const WeightView& W, int64_t n, int64_t nb, const ActView& A, int64_t m, float* y,
               int64_t ldy, hipStream_t s) {
  if (m <= 16) launch_t<TYPE, 1, NT, kWaves>(W, n, nb, A, m, y, ldy, s);
  else if (m <= 32) launch_t<TYPE, 2, NT, kWaves>(W, n, nb, A, m, y, ldy, s);
  else launch_t<TYPE, 4, NT, kWaves>(W, n, nb, A, m, y, ldy, s);
}

// Weight rows per workgroup (16 NT): each workgroup re-reads all m activation
// rows, so wide tiles save that traffic (Q4_K 14336 x 4096, m = 64: 31.7 us
// with 64 rows, 38.3 with 32, 57.7 with 16), but a short matrix then leaves
// CUs idle, so the tile narrows until the grid holds about 256 workgroups
// (Q4_K at m = 64 with 64 / 32 / 16 rows: 4096 x 14336 81.8 / 55.1 / 47.8
// us, 8192 x 8192 51.4 / 35.8 / 55.1, 6144 x 4096 30.5 / 21.2 / 30.7,
// 10240 x 4096 31.0 / 38.0 / 44.2). The results do not depend on it.
template <int TYPE>
void launch_type(const WeightView& W, int64_t n, int64_t nb, const ActView& A, int64_t m, float* y,
                 int64_t ldy, hipStream_t s) {
  if (n > 8192) launch_nt<TYPE, 4>(W, n, nb, A, m, y, ldy, s);
  else if (n > 4096) launch_nt<TYPE, 2>(W, n, nb, A, m, y, ldy, s);
  else launch_nt<TYPE, 1>(W, n, nb, A, m, y, ldy, s);
}

}  // namespace

hipError_t launch_gemm_small(int type, const void* wq, int64_t n, int64_t k, const void* xq, int64_t m,
                             float* y, int64_t ldy, hipStream_t s) {
  WeightView W;
  W.base = static_cast<const uint8_t*>(wq);
  W.row_bytes = row_bytes(type, k);
  W.hdr_bytes = header_bytes(type, k);
  const ActView A = make_act(xq, m, k);
  const int64_t nb = k / 32;
  switch (type) {
    case kQ4_0: launch_type<kQ4_0>(W, n, nb, A, m, y, ldy, s); break;
    case kQ8_0: launch_type<kQ8_0>(W, n, nb, A, m, y, ldy, s); break;
    case kQ4_0H: launch_type<kQ4_0H>(W, n, nb, A, m, y, ldy, s); break;
    default: launch_type<kQ4_K>(W, n, nb, A, m, y, ldy, s); break;
  }
  return hipGetLastError();
}

}  // namespace qblk
