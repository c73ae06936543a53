// Prefill-path product Y[m][n] = X * W^T with int8 matrix-core tiles.
//
// Dequantize-free: each 32-block's integer dot product is one
// v_mfma_i32_32x32x32_i8 over a 32x32 output tile (K = 32 is exactly one
// block) and the block scales are applied to the int32 tile in fp32 right
// after it ("llama.cpp 推理引擎", §6.4: scales outside the integer values;
// §5.5: Q4_K sub-block scale d*sc_j and min d_min*mn_j; §7.3: prefill is
// compute-bound).
//
// Per (m, n, block) the scale step is the binding cost (the matrix core does
// the 32x32x32 block in 32 cycles, the VALU needs 4 cycles per instruction
// for the tile's 16 values per lane), so it is cut to two FMAs:
//   * the int32 accumulator of each block MFMA starts from the bit pattern of
//     the float 1.5 * 2^23, so the result, read as fp32, is 1.5 * 2^23 + S
//     exactly (|S| < 2^22), and fma(F, sw, -1.5 * 2^23 * sw) = round(S * sw)
//     in one instruction - exact for Q4_K, whose sw = d * sc_j has at most 17
//     significant bits so that 1.5 * 2^23 * sw is an fp32 number;
//   * acc = fma(S * sw, sa, acc) applies the activation scale.
// The min terms (Q4_K: sum_b (sa*A)[m][b] * (d_min*mn_j)[n][b]; Q4_0, whose
// codes are nibble - 8: sum_b (sa*A)[m][b] * (-8*d)[n][b]) are an fp32 matrix
// product over blocks and run on the matrix cores (v_mfma_f32_32x32x2f32).
// Q4_0 / Q8_0 scales are full fp32, so their main step converts S exactly
// and takes three instructions.
//
// Data movement: K steps of 4 blocks with two LDS buffers. While step s is
// computed, the activation and weight codes of step s+1 stream into the other
// buffer by direct global-to-LDS loads (lane l of a wave instruction lands at
// +16 l), and its scales are loaded into registers and decoded into LDS
// after the compute. Rows are XOR-swizzled in 16-byte units so that the MFMA
// operand reads are free of bank conflicts.
//
// Operands: A = activation codes (rows m), B = weight codes (columns n). A
// lane holds 16 int8 of one row / column for one half of the block; the
// 4-bit weights are unpacked in registers to the same 0,2,4,6,1,3,5,7 order
// the activation codes are stored in, so A and B slots pair up element by
// element without byte permutes.
#include <type_traits>

#include "qblk_device.h"

namespace qblk {
namespace {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v16i __attribute__((ext_vector_type(16)));
typedef float v16f __attribute__((ext_vector_type(16)));

constexpr int BM = 128;        // activation rows per workgroup
constexpr int BN = 128;        // weight rows per workgroup
constexpr int KB = 4;          // 32-blocks per K step
// waves per workgroup: kWaves / kWavesN along M, kWavesN along N. Measured
// on MI355X (512 x 14336 x 4096): 4 waves of 32 x 128 are 4% faster than 2 x 2
// waves of 64 x 64 for Q4_K (half the activation-scale LDS reads per block)
// and 2% for Q8_0, 4% slower for Q4_0; 8 waves of 32 x 64 are 13% slower for
// Q4_K, whose scale step needs more registers.
constexpr int kWaves = 4;
constexpr int kWavesN = 1;
constexpr int TM = BM / 32 / (kWaves / kWavesN);  // 32-row MFMA tiles per wave
constexpr int TN = BN / 32 / kWavesN;             // 32-column MFMA tiles per wave
constexpr int kThreads = 64 * kWaves;
constexpr int kAInstr = BM * 8 / 64 / kWaves;     // activation DMA instructions per wave and stage
// kMagicBits / kMagic (fp32 1.5 * 2^23): qblk_device.h

// Min-term operands of a step in LDS (Q4_K: d_act * code sum and d_min * mn;
// Q4_0: d_act * code sum and -8 d); Q8_0 has no min term.
struct MinOps {
  float asc[KB][BM];  // d * (code sum)
  float wm[KB][BN];   // weight block min
};
struct NoMinOps {};

template <int TYPE>
struct Cfg {
  static constexpr int kWRow = TYPE == kQ8_0 ? 32 * KB : 16 * KB;  // weight bytes per row per step
  static constexpr bool kHasMin = TYPE != kQ8_0;
  using Min = std::conditional_t<kHasMin, MinOps, NoMinOps>;
};

// One LDS buffer: the codes of a K step (filled by direct loads) and its
// decoded scales.
template <int TYPE>
struct Stage {
  uint8_t a[BM * 32 * KB];       // activation codes, row r at 128 r, swizzled
  uint8_t w[BN * Cfg<TYPE>::kWRow];  // weight codes, row r at kWRow r, swizzled
  float sa[KB][BM];              // activation scale d
  float sw[KB][BN];              // weight block scale
  typename Cfg<TYPE>::Min mn;    // min-term operands (not for Q8_0: keeps its two
                                 // stages within half the CU's LDS)
};

// 16-byte unit positions inside a row (XOR swizzle)
__device__ __forceinline__ int a_pos(int r, int c) { return c ^ ((r >> 1) & 7); }  // 8 units per row
template <int TYPE>
__device__ __forceinline__ int w_pos(int r, int c) {
  if constexpr (TYPE == kQ8_0) return c ^ (r & 7);  // 8 units per row
  return c ^ ((r >> 2) & 3);                         // 4 units per row
}

// 16 bytes per lane from global memory straight into LDS; lane l of the wave
// writes lds_base + 16 l (lds_base must be wave-uniform).
__device__ __forceinline__ void lds_dma16(const uint8_t* src, uint8_t* lds_base) {
  __builtin_amdgcn_global_load_lds(src, lds_base, 16, 0, 0);
}

template <int TYPE>
struct GemmCtx {
  WeightView W;
  ActView A;
  int64_t n, nb, m, m0, n0;
};

// Per-lane sources of the direct loads, fixed for the launch: 32-bit byte
// offsets from the tile's first activation row / weight row (whose 64-bit
// addresses are wave-uniform), and the 16-byte unit of the step each load
// fills (a load is skipped when its unit lies past the last block).
template <int TYPE>
struct DmaLanes {
  static constexpr int kUnits = Cfg<TYPE>::kWRow / 16;  // weight units per row
  static constexpr int kInstr = BN * kUnits / 64 / kWaves;  // weight loads per wave
  const uint8_t* a_base;
  const uint8_t* w_base;
  uint32_t a_off[kAInstr];
  uint32_t w_off[kInstr];
  int a_unit[kAInstr];
  int w_unit[kInstr];
};

template <int TYPE>
__device__ __forceinline__ DmaLanes<TYPE> dma_lanes(const GemmCtx<TYPE>& g, int wave, int lane) {
  DmaLanes<TYPE> d;
  const int64_t k = g.nb * 32;
  d.a_base = g.A.q + g.m0 * k;
  d.w_base = g.W.base + g.n0 * g.W.row_bytes + g.W.hdr_bytes;
#pragma unroll
  for (int i = 0; i < kAInstr; ++i) {
    const int u = 64 * (kAInstr * wave + i) + lane;  // unit index in the stage
    const int r = u >> 3;
    d.a_unit[i] = a_pos(r, u & 7);  // global unit stored at this position
    const int64_t rr = g.m0 + r < g.m ? r : g.m - 1 - g.m0;
    d.a_off[i] = static_cast<uint32_t>(rr * k + 16 * d.a_unit[i]);
  }
#pragma unroll
  for (int i = 0; i < DmaLanes<TYPE>::kInstr; ++i) {
    const int u = 64 * (DmaLanes<TYPE>::kInstr * wave + i) + lane;
    const int r = u / DmaLanes<TYPE>::kUnits;
    d.w_unit[i] = w_pos<TYPE>(r, u % DmaLanes<TYPE>::kUnits);
    const int64_t rr = g.n0 + r < g.n ? r : g.n - 1 - g.n0;
    d.w_off[i] = static_cast<uint32_t>(rr * g.W.row_bytes + 16 * d.w_unit[i]);
  }
  return d;
}

// Direct global-to-LDS loads of step `st`'s codes into stage `S` (issued by
// every wave; each wave instruction writes 1 KiB of the stage).
template <int TYPE>
__device__ __forceinline__ void issue_codes(const GemmCtx<TYPE>& g, const DmaLanes<TYPE>& d,
                                            Stage<TYPE>* __restrict__ S, int64_t st, int wave) {
  const int64_t blk0 = st * KB;
  const int nblk = static_cast<int>(g.nb - blk0 < KB ? g.nb - blk0 : KB);
  const uint32_t a_step = static_cast<uint32_t>(32 * blk0);
  const uint32_t w_step = static_cast<uint32_t>((Cfg<TYPE>::kWRow / KB) * blk0);
  // activations: BM rows x 8 units = 16 instructions, kAInstr per wave
#pragma unroll
  for (int i = 0; i < kAInstr; ++i) {
    if (d.a_unit[i] < 2 * nblk)
      lds_dma16(d.a_base + (d.a_off[i] + a_step), S->a + 1024 * (kAInstr * wave + i));
  }
  // weights
  constexpr int kPerBlk = DmaLanes<TYPE>::kUnits / KB;  // units per block (1 or 2)
#pragma unroll
  for (int i = 0; i < DmaLanes<TYPE>::kInstr; ++i) {
    if (d.w_unit[i] < kPerBlk * nblk)
      lds_dma16(d.w_base + (d.w_off[i] + w_step),
                S->w + 1024 * (DmaLanes<TYPE>::kInstr * wave + i));
  }
}

// Scale data of step `st` into registers (decoded into LDS after the compute).
struct ScaleRegs {
  uint4 act;  // (d, sum) of two blocks of one activation row
  uint4 wgt;  // Q4_K header / four fp32 block scales of one weight row
};

// Per-thread scale sources, fixed for the launch: threads below 2 BM load
// the (d, sum) pairs of blocks 2h, 2h+1 of activation row tid/2; threads
// kWgtBase + i (i < BN) the header / scale region of weight row i.
constexpr int kWgtBase = kThreads >= 2 * BM + BN ? 2 * BM : 0;
__device__ __forceinline__ bool act_lane(int tid) { return tid < 2 * BM; }
__device__ __forceinline__ int wgt_row(int tid) { return tid - kWgtBase; }  // valid in [0, BN)
struct ScaleLanes {
  const uint8_t* act;
  const uint8_t* wgt;
};

template <int TYPE>
__device__ __forceinline__ ScaleLanes scale_lanes(const GemmCtx<TYPE>& g, int tid) {
  ScaleLanes l;
  const int r = (tid >> 1) & (BM - 1), h = tid & 1;
  const int64_t gm = g.m0 + r < g.m ? g.m0 + r : g.m - 1;
  l.act = g.A.ds + 8 * (gm * g.nb + 2 * h);
  const int wr = wgt_row(tid) & (BN - 1);
  const int64_t gn = g.n0 + wr < g.n ? g.n0 + wr : g.n - 1;
  l.wgt = g.W.row(gn);
  return l;
}

template <int TYPE>
__device__ __forceinline__ ScaleRegs load_scales(const GemmCtx<TYPE>& g, const ScaleLanes& sl,
                                                 int64_t st, int tid) {
  ScaleRegs s;
  const int64_t blk0 = st * KB;
  const int nblk = static_cast<int>(g.nb - blk0 < KB ? g.nb - blk0 : KB);
  const int h = tid & 1;  // blocks 2h, 2h+1
  // two 8-byte loads: a row's (d, sum) pairs are only 8-byte aligned, and the
  // second block may lie past the last block of the row
  const uint8_t* src = sl.act + 8 * blk0;
  uint2 p0 = make_uint2(0, 0), p1 = make_uint2(0, 0);
  if (act_lane(tid) && 2 * h < nblk) p0 = *reinterpret_cast<const uint2*>(src);
  if (act_lane(tid) && 2 * h + 1 < nblk) p1 = *reinterpret_cast<const uint2*>(src + 8);
  s.act = make_uint4(p0.x, p0.y, p1.x, p1.y);
  s.wgt = make_uint4(0, 0, 0, 0);
  if (wgt_row(tid) >= 0 && wgt_row(tid) < BN) {
    if constexpr (TYPE == kQ4_K) {
      s.wgt = load16(sl.wgt + 16 * (blk0 >> 3));
    } else if constexpr (TYPE == kQ4_0H) {
      // 8 bytes of fp16 scales; the padded header region keeps this in bounds
      const uint2 h = *reinterpret_cast<const uint2*>(sl.wgt + 2 * blk0);
      s.wgt = make_uint4(h.x, h.y, 0, 0);
    } else {
      // 16 bytes of scales; the padded header region keeps this in bounds
      s.wgt = load16(sl.wgt + 4 * blk0);
    }
  }
  return s;
}

template <int TYPE>
__device__ __forceinline__ void store_scales(Stage<TYPE>* __restrict__ S, const ScaleRegs& s, int64_t st,
                                             int tid) {
  const int r = tid >> 1;
  const int h = tid & 1;
  const float d0 = __uint_as_float(s.act.x), d1 = __uint_as_float(s.act.z);
  if (act_lane(tid)) {
    S->sa[2 * h][r] = d0;
    S->sa[2 * h + 1][r] = d1;
    if constexpr (Cfg<TYPE>::kHasMin) {
      S->mn.asc[2 * h][r] = d0 * static_cast<float>(static_cast<int>(s.act.y));
      S->mn.asc[2 * h + 1][r] = d1 * static_cast<float>(static_cast<int>(s.act.w));
    }
  }
  const int wr = wgt_row(tid);
  if (wr >= 0 && wr < BN) {
    if constexpr (TYPE == kQ4_K) {
      const float d = half_bits_to_float(s.wgt.x);
      const float dmin = half_bits_to_float(s.wgt.x >> 16);
      const int j0 = static_cast<int>((st * KB) & 7);
#pragma unroll
      for (int jj = 0; jj < KB; ++jj) {
        S->sw[jj][wr] = d * static_cast<float>(q4k_sc(s.wgt, j0 + jj));
        S->mn.wm[jj][wr] = dmin * static_cast<float>(q4k_mn(s.wgt, j0 + jj));
      }
    } else {
      float dw[4] = {__uint_as_float(s.wgt.x), __uint_as_float(s.wgt.y),
                     __uint_as_float(s.wgt.z), __uint_as_float(s.wgt.w)};
      if constexpr (TYPE == kQ4_0H) {
        dw[0] = half_bits_to_float(s.wgt.x);
        dw[1] = half_bits_to_float(s.wgt.x >> 16);
        dw[2] = half_bits_to_float(s.wgt.y);
        dw[3] = half_bits_to_float(s.wgt.y >> 16);
      }
#pragma unroll
      for (int jj = 0; jj < KB; ++jj) {
        S->sw[jj][wr] = dw[jj];
        if constexpr (Cfg<TYPE>::kHasMin) S->mn.wm[jj][wr] = -8.0f * dw[jj];  // Q4_0: nibble - 8
      }
    }
  }
}

struct Acc {
  v16f main[TM][TN];  // scale steps (VALU) and min terms (matrix core) accumulate here
};

// The MFMAs and scale steps of one K step from stage S.
template <int TYPE>
__device__ __forceinline__ void compute(const Stage<TYPE>* __restrict__ S, int nblk, int wm0, int wn0, int half,
                                        int l32, const v16i& cinit, Acc& acc) {
  for (int j = 0; j < nblk; ++j) {
    v4i bop[TN];
    float sw[TN], ncs[TN];
#pragma unroll
    for (int tn = 0; tn < TN; ++tn) {
      const int r = wn0 + 32 * tn + l32;
      if constexpr (TYPE == kQ8_0) {
        const uint4 w = *reinterpret_cast<const uint4*>(
            S->w + Cfg<TYPE>::kWRow * r + 16 * w_pos<TYPE>(r, 2 * j + half));
        bop[tn] = v4i{static_cast<int>(w.x), static_cast<int>(w.y), static_cast<int>(w.z),
                      static_cast<int>(w.w)};
      } else {
        const uint2 w = *reinterpret_cast<const uint2*>(
            S->w + Cfg<TYPE>::kWRow * r + 16 * w_pos<TYPE>(r, j) + 8 * half);
        const uint32_t msk = 0x0F0F0F0Fu;
        bop[tn] = v4i{static_cast<int>(w.x & msk), static_cast<int>((w.x >> 4) & msk),
                      static_cast<int>(w.y & msk), static_cast<int>((w.y >> 4) & msk)};
      }
      sw[tn] = S->sw[j][r];
      ncs[tn] = -kMagic * sw[tn];
    }
#pragma unroll
    for (int tm = 0; tm < TM; ++tm) {
      const int ra = wm0 + 32 * tm + l32;
      const uint4 a = *reinterpret_cast<const uint4*>(S->a + 128 * ra + 16 * a_pos(ra, 2 * j + half));
      const v4i aop = v4i{static_cast<int>(a.x), static_cast<int>(a.y), static_cast<int>(a.z),
                          static_cast<int>(a.w)};
      // activation scales of this lane's 16 rows: 4 consecutive rows per quarter
      float sa[16];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const float4 s4 =
            *reinterpret_cast<const float4*>(&S->sa[j][wm0 + 32 * tm + 8 * q + 4 * half]);
        sa[4 * q + 0] = s4.x;
        sa[4 * q + 1] = s4.y;
        sa[4 * q + 2] = s4.z;
        sa[4 * q + 3] = s4.w;
      }
#pragma unroll
      for (int tn = 0; tn < TN; ++tn) {
        const v16i c = __builtin_amdgcn_mfma_i32_32x32x32_i8(aop, bop[tn], cinit, 0, 0, 0);
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          float t;
          if constexpr (TYPE == kQ4_K) {
            t = fmaf(__int_as_float(c[v]), sw[tn], ncs[tn]);  // = round(S * sw)
          } else {
            t = static_cast<float>(c[v]) * sw[tn];
          }
          acc.main[tm][tn][v] = fmaf(t, sa[v], acc.main[tm][tn][v]);
        }
      }
    }
  }
  // min terms on the matrix cores: K = 2 blocks per instruction
  if constexpr (Cfg<TYPE>::kHasMin) {
#pragma unroll
    for (int i = 0; i < KB / 2; ++i) {
      if (2 * i < nblk) {  // uniform
        const int b = 2 * i + half;
        const bool okb = b < nblk;
        float af[TM], bf[TN];
#pragma unroll
        for (int tm = 0; tm < TM; ++tm) af[tm] = okb ? S->mn.asc[b][wm0 + 32 * tm + l32] : 0.0f;
#pragma unroll
        for (int tn = 0; tn < TN; ++tn) bf[tn] = okb ? S->mn.wm[b][wn0 + 32 * tn + l32] : 0.0f;
#pragma unroll
        for (int tm = 0; tm < TM; ++tm)
#pragma unroll
          for (int tn = 0; tn < TN; ++tn)
            acc.main[tm][tn] =
                __builtin_amdgcn_mfma_f32_32x32x2f32(af[tm], bf[tn], acc.main[tm][tn], 0, 0, 0);
      }
    }
  }
}

// One K step: the codes (and scales) of step st+1 stream into `nxt` while
// step st is computed from `cur`. `cur` and `nxt` are distinct LDS buffers;
// declaring them restrict lets the compiler see that the compute's LDS reads
// never wait for the direct loads into `nxt`.
template <int TYPE>
__device__ __forceinline__ bool step(const GemmCtx<TYPE>& g, const DmaLanes<TYPE>& dl,
                                     const ScaleLanes& sl,
                                     const Stage<TYPE>* __restrict__ cur,
                                     Stage<TYPE>* __restrict__ nxt, int64_t st, int64_t steps,
                                     int tid, int wave, int wm0, int wn0, int half,
                                     int l32, const v16i& cinit, Acc& acc) {
  __builtin_amdgcn_s_waitcnt(0);  // this wave's loads into `cur` are done
  __syncthreads();                // everyone's; the previous readers of `nxt` are done
  const bool more = st + 1 < steps;
  ScaleRegs sc;
  if (more) {
    // scale loads first: vmcnt retires in order, so waiting for them later
    // does not wait for the code loads issued after them
    sc = load_scales<TYPE>(g, sl, st + 1, tid);
    issue_codes<TYPE>(g, dl, nxt, st + 1, wave);
  }
  const int nblk = static_cast<int>(g.nb - st * KB < KB ? g.nb - st * KB : KB);
  compute<TYPE>(cur, nblk, wm0, wn0, half, l32, cinit, acc);
  if (more) {
    asm volatile("" ::: "memory");  // keep the scale stores after the compute
    store_scales<TYPE>(nxt, sc, st + 1, tid);
  }
  return more;
}

template <int TYPE>
__global__ __launch_bounds__(kThreads) void gemm_kernel(WeightView W, int64_t n, int64_t nb,
                                                        ActView A, int64_t m,
                                                        float* __restrict__ y, int64_t ldy) {
  __shared__ __attribute__((aligned(16))) Stage<TYPE> s0;
  __shared__ __attribute__((aligned(16))) Stage<TYPE> s1;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm0 = (wave / kWavesN) * (32 * TM);  // wave's row offset in the tile
  const int wn0 = (wave % kWavesN) * (32 * TN);  // wave's column offset in the tile
  const int half = lane >> 5;        // which 16 elements of a block this lane holds
  const int l32 = lane & 31;

  GemmCtx<TYPE> g;
  g.W = W;
  g.A = A;
  g.n = n;
  g.nb = nb;
  g.m = m;
  g.m0 = static_cast<int64_t>(blockIdx.y) * BM;
  g.n0 = static_cast<int64_t>(blockIdx.x) * BN;

  Acc acc;
#pragma unroll
  for (int a = 0; a < TM; ++a)
#pragma unroll
    for (int b = 0; b < TN; ++b)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc.main[a][b][v] = 0.0f;
  v16i cinit;
#pragma unroll
  for (int v = 0; v < 16; ++v) cinit[v] = TYPE == kQ4_K ? kMagicBits : 0;

  const int64_t steps = (nb + KB - 1) / KB;
  // prologue: step 0 into s0
  const ScaleLanes sl = scale_lanes<TYPE>(g, tid);
  store_scales<TYPE>(&s0, load_scales<TYPE>(g, sl, 0, tid), 0, tid);
  const DmaLanes<TYPE> dl = dma_lanes<TYPE>(g, wave, lane);
  issue_codes<TYPE>(g, dl, &s0, 0, wave);

  for (int64_t st = 0; st < steps; st += 2) {
    if (!step<TYPE>(g, dl, sl, &s0, &s1, st, steps, tid, wave, wm0, wn0, half, l32, cinit, acc))
      break;
    if (!step<TYPE>(g, dl, sl, &s1, &s0, st + 1, steps, tid, wave, wm0, wn0, half, l32, cinit,
                    acc))
      break;
  }

  // ---- store: lane holds column n = l32 and 16 rows of each 32 x 32 tile
#pragma unroll
  for (int tm = 0; tm < TM; ++tm)
#pragma unroll
    for (int tn = 0; tn < TN; ++tn) {
      const int64_t gn = g.n0 + wn0 + 32 * tn + l32;
      if (gn >= n) continue;
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int64_t gm = g.m0 + wm0 + 32 * tm + 8 * (v >> 2) + 4 * half + (v & 3);
        if (gm < m) y[gm * ldy + gn] = acc.main[tm][tn][v];
      }
    }
}

// K split over two groups of four waves (a grid of at most one workgroup per
// CU would otherwise run one wave per SIMD): group 0 takes the first half of
// the K steps, group 1 the second, each with its own two stages; then group
// 1's partial tiles pass through LDS and group 0 adds them to its own (in
// that order) and stores. Both groups run the same number of steps (the
// shorter one idles through its last), so their barriers pair up.
template <int TYPE>
__device__ __forceinline__ void step_ks(const GemmCtx<TYPE>& g, const DmaLanes<TYPE>& dl, const ScaleLanes& sl,
                                        const Stage<TYPE>* __restrict__ cur, Stage<TYPE>* __restrict__ nxt,
                                        int64_t st, int64_t send, bool active, int ltid, int lwave, int wm0,
                                        int wn0, int half, int l32, const v16i& cinit, Acc& acc) {
  __builtin_amdgcn_s_waitcnt(0);  // this wave's loads into `cur` are done
  __syncthreads();                // everyone's; the previous readers of `nxt` are done
  if (!active) return;            // uniform over the group
  const bool more = st + 1 < send;
  ScaleRegs sc;
  if (more) {
    sc = load_scales<TYPE>(g, sl, st + 1, ltid);
    issue_codes<TYPE>(g, dl, nxt, st + 1, lwave);
  }
  const int nblk = static_cast<int>(g.nb - st * KB < KB ? g.nb - st * KB : KB);
  compute<TYPE>(cur, nblk, wm0, wn0, half, l32, cinit, acc);
  if (more) {
    asm volatile("" ::: "memory");
    store_scales<TYPE>(nxt, sc, st + 1, ltid);
  }
}

template <int TYPE>
__global__ __launch_bounds__(2 * kThreads) void gemm_ksplit_kernel(WeightView W, int64_t n, int64_t nb,
                                                                   ActView A, int64_t m,
                                                                   float* __restrict__ y, int64_t ldy) {
  __shared__ __attribute__((aligned(16))) Stage<TYPE> stg[2][2];  // [K half][buffer]
  static_assert(sizeof(float) * kWaves * TM * TN * 16 * 64 <= 2 * sizeof(Stage<TYPE>),
                "group 1's partial tiles fit group 0's two stages");

  const int tid = threadIdx.x;
  const int grp = __builtin_amdgcn_readfirstlane(tid / kThreads);  // K half
  const int ltid = tid % kThreads;
  const int lane = tid & 63;
  const int lwave = __builtin_amdgcn_readfirstlane(ltid >> 6);
  const int wm0 = (lwave / kWavesN) * (32 * TM);
  const int wn0 = (lwave % kWavesN) * (32 * TN);
  const int half = lane >> 5;
  const int l32 = lane & 31;

  GemmCtx<TYPE> g;
  g.W = W;
  g.A = A;
  g.n = n;
  g.nb = nb;
  g.m = m;
  g.m0 = static_cast<int64_t>(blockIdx.y) * BM;
  g.n0 = static_cast<int64_t>(blockIdx.x) * BN;

  Acc acc;
#pragma unroll
  for (int a = 0; a < TM; ++a)
#pragma unroll
    for (int b = 0; b < TN; ++b)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc.main[a][b][v] = 0.0f;
  v16i cinit;
#pragma unroll
  for (int v = 0; v < 16; ++v) cinit[v] = TYPE == kQ4_K ? kMagicBits : 0;

  const int64_t steps = (nb + KB - 1) / KB;  // the launcher guarantees at least 2
  const int64_t hsteps = (steps + 1) / 2;
  const int64_t sbeg = grp ? hsteps : 0, send = grp ? steps : hsteps;
  const ScaleLanes sl = scale_lanes<TYPE>(g, ltid);
  const DmaLanes<TYPE> dl = dma_lanes<TYPE>(g, lwave, lane);
  store_scales<TYPE>(&stg[grp][0], load_scales<TYPE>(g, sl, sbeg, ltid), sbeg, ltid);
  issue_codes<TYPE>(g, dl, &stg[grp][0], sbeg, lwave);

  for (int64_t i = 0; i < hsteps; ++i) {
    const int64_t st = sbeg + i;
    const bool active = st < send;
    if (i & 1)
      step_ks<TYPE>(g, dl, sl, &stg[grp][1], &stg[grp][0], st, send, active, ltid, lwave, wm0, wn0, half, l32,
                    cinit, acc);
    else
      step_ks<TYPE>(g, dl, sl, &stg[grp][0], &stg[grp][1], st, send, active, ltid, lwave, wm0, wn0, half, l32,
                    cinit, acc);
  }

  // group 1's partial tiles to group 0, through group 0's stages
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  float* red = reinterpret_cast<float*>(&stg[0][0]);
  if (grp == 1) {
#pragma unroll
    for (int tm = 0; tm < TM; ++tm)
#pragma unroll
      for (int tn = 0; tn < TN; ++tn)
#pragma unroll
        for (int v = 0; v < 16; ++v) red[(((lwave * TM + tm) * TN + tn) * 16 + v) * 64 + lane] = acc.main[tm][tn][v];
  }
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  if (grp == 0) {
#pragma unroll
    for (int tm = 0; tm < TM; ++tm)
#pragma unroll
      for (int tn = 0; tn < TN; ++tn) {
        const int64_t gn = g.n0 + wn0 + 32 * tn + l32;
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const float val = acc.main[tm][tn][v] + red[(((lwave * TM + tm) * TN + tn) * 16 + v) * 64 + lane];
          const int64_t gm = g.m0 + wm0 + 32 * tm + 8 * (v >> 2) + 4 * half + (v & 3);
          if (gn < n && gm < m) y[gm * ldy + gn] = val;
        }
      }
  }
}

}  // namespace

hipError_t launch_gemm(int type, const void* wq, int64_t n, int64_t k, const void* xq, int64_t m,
                       float* y, int64_t ldy, hipStream_t s) {
  if (gemm_few_rows(n, m)) return launch_gemm_small(type, wq, n, k, xq, m, y, ldy, s);
  WeightView W;
  W.base = static_cast<const uint8_t*>(wq);
  W.row_bytes = row_bytes(type, k);
  W.hdr_bytes = header_bytes(type, k);
  const ActView A = make_act(xq, m, k);
  const int64_t nb = k / 32;
  const dim3 grid(static_cast<uint32_t>((n + BN - 1) / BN), static_cast<uint32_t>((m + BM - 1) / BM));
  if (gemm_split_k(n, k, m)) {
    switch (type) {
      case kQ4_0: hipLaunchKernelGGL(gemm_ksplit_kernel<kQ4_0>, grid, dim3(2 * kThreads), 0, s, W, n, nb, A, m, y, ldy); break;
      case kQ8_0: hipLaunchKernelGGL(gemm_ksplit_kernel<kQ8_0>, grid, dim3(2 * kThreads), 0, s, W, n, nb, A, m, y, ldy); break;
      case kQ4_0H: hipLaunchKernelGGL(gemm_ksplit_kernel<kQ4_0H>, grid, dim3(2 * kThreads), 0, s, W, n, nb, A, m, y, ldy); break;
      default: hipLaunchKernelGGL(gemm_ksplit_kernel<kQ4_K>, grid, dim3(2 * kThreads), 0, s, W, n, nb, A, m, y, ldy); break;
    }
    return hipGetLastError();
  }
  switch (type) {
    case kQ4_0: hipLaunchKernelGGL(gemm_kernel<kQ4_0>, grid, dim3(kThreads), 0, s, W, n, nb, A, m, y, ldy); break;
    case kQ8_0: hipLaunchKernelGGL(gemm_kernel<kQ8_0>, grid, dim3(kThreads), 0, s, W, n, nb, A, m, y, ldy); break;
    case kQ4_0H: hipLaunchKernelGGL(gemm_kernel<kQ4_0H>, grid, dim3(kThreads), 0, s, W, n, nb, A, m, y, ldy); break;
    default: hipLaunchKernelGGL(gemm_kernel<kQ4_K>, grid, dim3(kThreads), 0, s, W, n, nb, A, m, y, ldy); break;
  }
  return hipGetLastError();
}

}  // namespace qblk
