// Decode-path product y[b][n] = sum_j scale * intdot(block j), few activation
// rows. HBM-bound: every packed weight byte is read exactly once.
//
// Integer dot inside each 32-block, fp32 scales outside it ("llama.cpp 推理
// 引擎", §6.4; wmrh.cn "bare engine" article, §2.2 int4 x int8 dot); Q4_K
// sub-block scale d*sc_j and min d_min*mn_j per §5.5. Decode streams every
// weight once per token, so the kernel is bound by HBM bandwidth ("llama.cpp
// 推理引擎", §7.3; "llama.cpp：一个人、一个周末…", section 3).
//
// Mapping: one wave per R weight rows. Lane l takes 32-blocks l, l+64, ...;
// one 16-byte load per lane then covers 64 consecutive blocks of 4-bit codes
// (a "chunk"): each wave load is a contiguous KiB of a row. A wave issues the
// loads of U chunks (weights, scales, activations) before any arithmetic, so
// U*R KiB per wave are in flight; the activation codes are reused for the R
// rows. Row bases are wave-uniform (scalar registers) and lane offsets 32-bit,
// so loads need no per-lane 64-bit address arithmetic. Per block:
// v_dot4_i32_i8 on unpacked nibbles (or int8 codes), then one or two fp32 FMAs
// with the block scales; a DPP wave reduction at the end.
#include <atomic>

#include "qblk_device.h"

namespace qblk {
namespace {

constexpr int kWavesPerBlock = 4;

template <int TYPE>
struct WChunk;  // one lane's weight codes for one block
template <>
struct WChunk<kQ4_0> { uint4 q; };
template <>
struct WChunk<kQ4_K> { uint4 q; };
template <>
struct WChunk<kQ8_0> { uint4 q0, q1; };
template <>
struct WChunk<kQ4_0H> { uint4 q; };

template <int TYPE>
struct WScale;  // one lane's block scale data
template <>
struct WScale<kQ4_0> { float d; };
template <>
struct WScale<kQ8_0> { float d; };
template <>
struct WScale<kQ4_K> { uint4 h; };
template <>
struct WScale<kQ4_0H> { float d; };

// Loads of one lane's block `blk` of a row whose (wave-uniform) base is in
// scalar registers: 32-bit lane offsets let the loads use a scalar base.
template <int TYPE>
__device__ __forceinline__ void load_block(const uint8_t* __restrict__ wrow, uint32_t hdr_bytes,
                                           uint32_t blk, WChunk<TYPE>& w, WScale<TYPE>& s) {
  if constexpr (TYPE == kQ4_K) {
    s.h = load16(wrow + 16u * (blk >> 3));
    w.q = load_stream16(wrow + (hdr_bytes + 16u * blk));
  } else if constexpr (TYPE == kQ4_0) {
    s.d = __uint_as_float(load_stream4(wrow + 4u * blk));
    w.q = load_stream16(wrow + (hdr_bytes + 16u * blk));
  } else if constexpr (TYPE == kQ4_0H) {
    s.d = half_bits_to_float(load_stream2(wrow + 2u * blk));
    w.q = load_stream16(wrow + (hdr_bytes + 16u * blk));
  } else {
    s.d = __uint_as_float(load_stream4(wrow + 4u * blk));
    w.q0 = load_stream16(wrow + (hdr_bytes + 32u * blk));
    w.q1 = load_stream16(wrow + (hdr_bytes + 32u * blk + 16u));
  }
}

// Kernel arguments: plain pointers and sizes; row bases are made
// wave-uniform so that they live in scalar registers.
struct GemvArgs {
  const uint8_t* w;    // packed rows
  int64_t row_bytes;
  uint32_t hdr_bytes;
  int64_t n;           // rows
  uint32_t nb;         // 32-blocks per row
  const uint8_t* aq;   // activation codes [B][k]      (unfused)
  const uint8_t* ads;  // activation (d, sum) [B][nb]  (unfused)
  const float* x;      // fp32 activations [B][ldx]    (fused)
  int64_t ldx;
  float* y;
  int64_t ldy;
  // in-kernel quantization handoff (SYNC variants): the first workgroups
  // quantize 64-block slices of x into the workspace activation buffer
  // (aq/ads alias it) and tag each slice in 8 flag copies
  uint8_t* xq_codes;
  uint8_t* xq_ds;
  uint64_t* flags;     // [8][flag_stride] u64
  uint32_t nslices;    // ceil(nb / 64) slices per activation row
  uint32_t flag_stride;
  uint32_t* fallbacks; // counter of workgroups that gave up waiting
  uint64_t wait_ticks; // the wait bound, 100 MHz ticks
};

// ---------------------------------------------------------------- in-kernel handoff
// A launch-unique tag: the dispatch id of the packet (counts dispatches per
// hardware queue) mixed with the packet's address (which identifies the
// queue), so a flag left in the workspace by an earlier launch never matches.
extern "C" __device__ uint64_t qblk_llvm_dispatch_id() __asm("llvm.amdgcn.dispatch.id");

__device__ __forceinline__ uint64_t launch_tag() {
  const uint64_t id = qblk_llvm_dispatch_id();
  const uint64_t p = reinterpret_cast<uint64_t>(__builtin_amdgcn_dispatch_ptr());
  return (id * 0x9E3779B97F4A7C15ull) ^ (p << 1) ^ 1ull;  // never 0 for a zeroed workspace
}

// Workgroup quantizes slice `sl` (blocks 64*sl .. 64*sl+63) of the B rows
// of x into the workspace activation buffer with the qblk_quantize_act
// arithmetic: one block per quad of threads, 8 elements per thread. The
// stores are agent-scope atomic stores, which the L2 writes through to
// memory, so they are visible to every XCD once complete.
// Slice sl covers blocks 64 (sl mod nslices) .. +63 of activation row
// sl / nslices: one slice per workgroup-sized piece of work whatever the
// batch, so a larger batch spreads over more producers instead of making each
// one slower.
__device__ __forceinline__ void quantize_slice(const GemvArgs& g, uint32_t sl) {
  const uint32_t b = sl / g.nslices;
  const uint32_t blk = ((sl - b * g.nslices) << 6) + (threadIdx.x >> 2);
  const uint32_t sub = threadIdx.x & 3;
  if (threadIdx.x >= 256u || blk >= g.nb) return;  // whole quads; 64 blocks per slice
  const uint32_t k = g.nb * 32u;
  const float* src = g.x + b * g.ldx + 32u * blk + 8u * sub;
  const float4 v0 = *reinterpret_cast<const float4*>(src);
  const float4 v1 = *reinterpret_cast<const float4*>(src + 4);
  const float e[8] = {v0.x, v0.y, v0.z, v0.w, v1.x, v1.y, v1.z, v1.w};
  const Q8Group q = quantize_group8(e);
  __hip_atomic_store(reinterpret_cast<uint64_t*>(g.xq_codes + b * k + 32u * blk + 8u * sub),
                     static_cast<uint64_t>(q.codes.x) | static_cast<uint64_t>(q.codes.y) << 32,
                     __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  if (sub == 0)
    __hip_atomic_store(reinterpret_cast<uint64_t*>(g.xq_ds + 8u * (b * g.nb + blk)),
                       static_cast<uint64_t>(__float_as_uint(q.d)) |
                           static_cast<uint64_t>(static_cast<uint32_t>(q.sum)) << 32,
                       __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Producer side: workgroups below nslices quantize slices wg, wg + grid, ...
// and publish each. Every wave waits until its (write-through) stores have
// completed, the workgroup meets at a barrier, then one wave stores the
// slice's tag into each of the 8 flag copies. This is the hardware form of
// release ordering for atomic stores; a release fence would in addition
// write back the whole L2 of the XCD, which nothing here needs and which
// took 3-5 us per launch on MI355X while the weight stream was running.
template <int B>
__device__ __forceinline__ void produce(const GemvArgs& g, uint64_t tag) {
  for (uint32_t sl = blockIdx.x; sl < B * g.nslices; sl += gridDim.x) {
    quantize_slice(g, sl);
    __builtin_amdgcn_s_waitcnt(0);  // this wave's stores have completed
    __syncthreads();
    if (threadIdx.x < 8)
      __hip_atomic_store(g.flags + threadIdx.x * g.flag_stride + sl, tag, __ATOMIC_RELAXED,
                         __HIP_MEMORY_SCOPE_AGENT);
  }
}

// Consumer side: the workgroup polls the flag copy of its index mod 8 (one
// relaxed load per slice, spread over its threads) until every slice carries
// this launch's tag. Activation codes are read only after that, so no cache
// holds a line of them from before this launch (the kernel start invalidated
// the caches). The wait is bounded (20 ms unless a test lowers it): past the
// bound the workgroup counts itself in the workspace's fallback counter and
// quantizes every slice itself (the same bytes the producers write), so the
// kernel finishes with the right result even if the producers were never
// scheduled. All exits are decided by workgroup-wide reductions.
template <int B, int WAVES = 4>
__device__ __forceinline__ void wait_slices(const GemvArgs& g, uint64_t tag) {
  const uint64_t* f = g.flags + (blockIdx.x & 7u) * g.flag_stride;
  const uint64_t t0 = __builtin_amdgcn_s_memrealtime();
  while (true) {
    int pending = 0;
    for (uint32_t sl = threadIdx.x; sl < B * g.nslices; sl += 64u * WAVES)
      pending |= __hip_atomic_load(f + sl, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) != tag;
    if (!__syncthreads_or(pending)) return;
    const int late = __builtin_amdgcn_s_memrealtime() - t0 > g.wait_ticks;  // 100 MHz clock
    if (__syncthreads_or(late)) break;
  }
  if (threadIdx.x == 0)
    __hip_atomic_fetch_add(g.fallbacks, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  for (uint32_t sl = 0; sl < B * g.nslices; ++sl) quantize_slice(g, sl);
  __threadfence();
  __syncthreads();
}

// The per-block arithmetic of one weight row against B activation rows, in
// one fixed order for every kernel variant (so that all variants, fused or
// not, produce bit-identical results): integer dot of the 32 codes, then the
// fp32 scale FMAs, accumulated per lane in ascending block order.
template <int TYPE, int B, int U>
__device__ __forceinline__ void block_fma(uint32_t lane, const WChunk<TYPE>& w,
                                          const WScale<TYPE>& s, const uint4 (&a)[B][U][2],
                                          const float2 (&ds)[B][U], int u, float (&acc)[B]) {
  if constexpr (TYPE == kQ4_K) {
    // sw = d*sc_j has at most 17 significant bits, so -1.5*2^23*sw is an
    // fp32 number and fma(1.5*2^23 + S, sw, -1.5*2^23*sw) = round(S*sw), one
    // instruction; then the activation scale and the min term, whose
    // d_act*A is shared by the wave's rows
    const int j = static_cast<int>(lane & 7);  // sub-block inside the super-block
    const float sw = half_bits_to_float(s.h.x) * static_cast<float>(q4k_sc(s.h, j));
    const float wm = half_bits_to_float(s.h.x >> 16) * static_cast<float>(q4k_mn(s.h, j));
    const float ncs = -kMagic * sw;
#pragma unroll
    for (int b = 0; b < B; ++b) {
      const float t = fmaf(dot_nib32_magic(w.q, a[b][u][0], a[b][u][1]), sw, ncs);
      const float dA = ds[b][u].x * static_cast<float>(__float_as_int(ds[b][u].y));
      acc[b] = fmaf(wm, dA, fmaf(t, ds[b][u].x, acc[b]));
    }
  } else if constexpr (TYPE == kQ4_0 || TYPE == kQ4_0H) {
#pragma unroll
    for (int b = 0; b < B; ++b) {
      const int S = dot_nib32(w.q, a[b][u][0], a[b][u][1]) - 8 * __float_as_int(ds[b][u].y);
      acc[b] = fmaf(s.d * ds[b][u].x, static_cast<float>(S), acc[b]);
    }
  } else {
#pragma unroll
    for (int b = 0; b < B; ++b) {
      const int S = dot_i8x32(w.q0, w.q1, a[b][u][0], a[b][u][1]);
      acc[b] = fmaf(s.d * ds[b][u].x, static_cast<float>(S), acc[b]);
    }
  }
}

// ---------------------------------------------------------------- activation staging
// A workgroup copies the B rows' activation buffer into LDS once, so the
// waves read their 40 bytes per block and row from LDS rather than from L2
// for every group of R rows. LDS layout per activation row (stride
// act_lds_row(nb), whole 2 KiB chunks): for chunk c, the first 16 code bytes
// of its 64 blocks, then the second 16 (a lane's 16-B read is then
// contiguous with its neighbours', free of bank conflicts); after the B rows
// of codes the (d, sum) pairs, [B][nb].
// (act_lds_row, act_lds_bytes and the staging limits: qblk_internal.h)

template <int B, int WAVES = 4>
__device__ __forceinline__ void stage_acts(const GemvArgs& g, uint8_t* smem) {
  const uint32_t k = g.nb * 32u, kp = act_lds_row(g.nb);
#pragma unroll
  for (int b = 0; b < B; ++b) {
    for (uint32_t u = threadIdx.x; u < k / 16u; u += 64u * WAVES) {
      const uint32_t blk = u >> 1, h = u & 1u;
      *reinterpret_cast<uint4*>(smem + b * kp + (((blk >> 6) * 2u + h) << 10) + ((blk & 63u) << 4)) =
          load16(g.aq + b * k + 16u * u);
    }
  }
  uint8_t* sds = smem + B * kp;
  for (uint32_t i = threadIdx.x; i < B * g.nb; i += 64u * WAVES)
    *reinterpret_cast<uint2*>(sds + 8u * i) = *reinterpret_cast<const uint2*>(g.ads + 8u * i);
}

// One lane's activation data of block `blk` for the B rows, from LDS
// (ALDS) or from the global activation buffer.
template <int B, int U, bool ALDS>
__device__ __forceinline__ void load_act_block(const GemvArgs& g, const uint8_t* smem, uint32_t blk,
                                               int u, uint4 (&a)[B][U][2], float2 (&ds)[B][U]) {
  const uint32_t k = g.nb * 32u;
#pragma unroll
  for (int b = 0; b < B; ++b) {
    if constexpr (ALDS) {
      const uint8_t* ap = smem + b * act_lds_row(g.nb) + (((blk >> 6) * 2u) << 10) + ((blk & 63u) << 4);
      a[b][u][0] = *reinterpret_cast<const uint4*>(ap);
      a[b][u][1] = *reinterpret_cast<const uint4*>(ap + 1024);
      ds[b][u] = *reinterpret_cast<const float2*>(smem + B * act_lds_row(g.nb) + 8u * (b * g.nb + blk));
    } else {
      const uint8_t* ap = g.aq + b * k;
      a[b][u][0] = load16(ap + 32u * blk);
      a[b][u][1] = load16(ap + (32u * blk + 16u));
      ds[b][u] = *reinterpret_cast<const float2*>(g.ads + 8u * (b * g.nb) + 8u * blk);
    }
  }
}

// Classic variant: each wave issues the loads of U chunks for its R rows,
// then computes them; occupancy hides the latency. Best for large matrices.
// SYNC: the activation is quantized inside the launch (produce /
// wait_slices); ALDS: it is read from LDS (stage_acts). Either way the first
// chunks' weight loads are issued before the wait / staging.
// `block` is the workgroup's index within this product (blockIdx.x, or its
// offset inside a descriptor's range for the multi-product launch).
template <int TYPE, int B, int R, int U, bool SYNC, bool ALDS, int WAVES = kWavesPerBlock>
__device__ __forceinline__ void gemv_body(const GemvArgs& g, uint32_t block) {
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
  constexpr bool kAllWaves = SYNC || ALDS;  // workgroup barriers ahead: no early exit
  const uint32_t lane = threadIdx.x & 63;
  const int64_t wave = static_cast<int64_t>(block) * WAVES +
                       __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x >> 6));
  const int64_t row0 = wave * R;
  uint64_t tag = 0;
  if constexpr (SYNC) {
    tag = launch_tag();
    produce<B>(g, tag);
  }
  if constexpr (!kAllWaves) {
    if (row0 >= g.n) return;  // whole wave
  }
  const bool active = !kAllWaves || row0 < g.n;
  const uint8_t* wrow[R];
#pragma unroll
  for (int r = 0; r < R; ++r) {
    const int64_t rr = row0 + r < g.n ? row0 + r : g.n - 1;
    wrow[r] = g.w + rr * g.row_bytes;
  }
  const uint32_t nchunks = (g.nb + 63u) >> 6;

  float acc[R][B];
#pragma unroll
  for (int r = 0; r < R; ++r)
#pragma unroll
    for (int b = 0; b < B; ++b) acc[r][b] = 0.0f;

  auto load_weights = [&](uint32_t c0, WChunk<TYPE>(&w)[R][U], WScale<TYPE>(&s)[R][U]) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const uint32_t blk = ((c0 + u) << 6) + lane;
      if (active && blk < g.nb) {
#pragma unroll
        for (int r = 0; r < R; ++r) load_block<TYPE>(wrow[r], g.hdr_bytes, blk, w[r][u], s[r][u]);
      }
    }
  };
  auto load_acts = [&](uint32_t c0, int u, uint4(&a)[B][U][2], float2(&ds)[B][U]) {
    const uint32_t blk = ((c0 + u) << 6) + lane;
    if (blk < g.nb) load_act_block<B, U, ALDS>(g, smem, blk, u, a, ds);
  };
  auto compute = [&](uint32_t c0, const WChunk<TYPE>(&w)[R][U], const WScale<TYPE>(&s)[R][U],
                     const uint4(&a)[B][U][2], const float2(&ds)[B][U]) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const uint32_t blk = ((c0 + u) << 6) + lane;
      if (blk < g.nb) {
#pragma unroll
        for (int r = 0; r < R; ++r) block_fma<TYPE, B>(lane, w[r][u], s[r][u], a, ds, u, acc[r]);
      }
    }
  };

  uint32_t c_start = 0;
  if constexpr (kAllWaves) {
    // first U chunks: weight loads in flight while the activation is
    // awaited / staged; with the in-launch handoff and at most 2 rows per
    // wave, the next U chunks too (measured: 0.3 us less on the 70B q/k/v
    // and o launches; with 4 rows per wave the extra registers cost more)
    constexpr bool kPre2 = SYNC && R <= 2;
    WChunk<TYPE> w[R][U];
    WScale<TYPE> s[R][U];
    load_weights(0, w, s);
    WChunk<TYPE> w2[R][U];
    WScale<TYPE> s2[R][U];
    if constexpr (kPre2) load_weights(U, w2, s2);
    if constexpr (SYNC) wait_slices<B, WAVES>(g, tag);
    if constexpr (ALDS) {
      stage_acts<B, WAVES>(g, smem);
      __syncthreads();
    }
    if (!active) return;
    uint4 a[B][U][2];
    float2 ds[B][U];
#pragma unroll
    for (int u = 0; u < U; ++u) load_acts(0, u, a, ds);
    compute(0, w, s, a, ds);
    c_start = U;
    if constexpr (kPre2) {
#pragma unroll
      for (int u = 0; u < U; ++u) load_acts(U, u, a, ds);
      compute(U, w2, s2, a, ds);
      c_start = 2 * U;
    }
  }
  for (uint32_t c0 = c_start; c0 < nchunks; c0 += U) {
    WChunk<TYPE> w[R][U];
    WScale<TYPE> s[R][U];
    uint4 a[B][U][2];
    float2 ds[B][U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const uint32_t blk = ((c0 + u) << 6) + lane;
      if (blk < g.nb) {
#pragma unroll
        for (int r = 0; r < R; ++r) load_block<TYPE>(wrow[r], g.hdr_bytes, blk, w[r][u], s[r][u]);
      }
      load_acts(c0, u, a, ds);
    }
    compute(c0, w, s, a, ds);
  }

#pragma unroll
  for (int r = 0; r < R; ++r) {
#pragma unroll
    for (int b = 0; b < B; ++b) {
      const float v = wave_sum_dpp(acc[r][b]);
      if (lane == 63 && row0 + r < g.n) g.y[b * g.ldy + row0 + r] = v;
    }
  }
}

template <int TYPE, int B, int R, int U, bool SYNC = false, bool ALDS = false, int WAVES = kWavesPerBlock>
__global__ __launch_bounds__(64 * WAVES) void gemv_kernel(GemvArgs g) {
  gemv_body<TYPE, B, R, U, SYNC, ALDS, WAVES>(g, blockIdx.x);
}

// ---------------------------------------------------------------- matrix-core form, 2-8 activation rows
// Q4_K with 2 to 8 activation rows and k a multiple of 2048. The dot4 form
// spends 73 VALU instructions per row and block at 4 rows (32 of them
// dot4); here each block's integer dots run on v_mfma_i32_16x16x64_i8 and
// the VALU keeps the unpack, the scale decode and the scale FMAs (about 40).
//
// Operands (D = A x B, 16 x 16, K = 64): B holds 16 weight rows (column i =
// lane & 15), its k-group q = lane >> 4 holds half of block 4u + q of the
// step (two MFMAs per block pair of halves). A row m = 4 b + a (activation
// row a of a group of four, block b of the step) is nonzero only in k-group
// b, so output D[4 q + a][i] is the integer dot of weight row i with
// activation row a over one whole block: lane (i, q) ends with the four
// activation rows of its own row and block, whose scales it decoded itself
// (5-8 rows: a second group, two more MFMAs on the same B operand). A
// quarter of the MFMA work is useful; the matrix cores have that to spare.
//
// Data movement: that operand layout needs 16 rows per load, and 16-row
// loads of 64 bytes each stream at about two thirds of the bandwidth of the
// per-row KiB loads (a stream probe over the 70B gate/up: 4.4 against 6.4
// TB/s). So a workgroup owns one 16-row tile, and each 64-block chunk of its
// 16 rows (1 KiB per row, the row's headers, and the chunk's activation
// codes and scale pairs) moves by direct global-to-LDS loads into one of two
// LDS stages while the other is computed. Row r's lane l fetches block
// l ^ (r & 15) of the chunk, which keeps every load a whole KiB and makes the
// transposed operand reads conflict-free. The headers and activation units
// are permuted the same way (each lane fetches the unit that its LDS slot
// should hold): row r's header of super-block s sits at unit s ^ ((r >> 1) &
// 7), and activation slot a's 16-B unit U at U ^ ((a & 1) | (a & 2) << 2), so
// that the 16 lanes of each read hit 16 different bank groups (with the
// plain layouts, bank conflicts took about half of the LDS cycles; the 70B
// q/k/v at 4 rows went from 15.8 to 15.1 us). The four waves take 16 blocks of a
// chunk each; their sums meet in LDS at the end in wave order. The direct
// loads are issued by inline assembly with explicit waits: the compiler does
// not track them, and with its own waits every LDS read would drain the
// ring. Nothing else in the loop touches vector memory.
constexpr uint32_t kRingW = 16384;   // 16 rows x 1 KiB of codes
constexpr uint32_t kRingH = 2048;    // 16 rows x 128 B of headers
constexpr uint32_t kRingZero = 512;  // zero operand slots of the unused A lanes
// A stage holds the weights, the headers, then NA activation slots (4 for up
// to 4 rows, 8 for 5-8; slot a holds activation row min(a, rows - 1)): NA x
// 2 KiB of codes, then NA x 64 (d, sum) pairs. Two stages, then the zero
// slots; the tile-walking kernel adds one tile's partial sums, [4 waves][NA][16].
template <int NA>
struct RingLayout {
  static constexpr uint32_t kA = kRingW + kRingH;
  static constexpr uint32_t kD = kA + NA * 2048u;
  static constexpr uint32_t kStage = kD + NA * 512u;
  static constexpr uint32_t kZero = 2 * kStage;
  static constexpr uint32_t kLds = kZero + kRingZero;
  static constexpr uint32_t kPart = kLds;
  static constexpr uint32_t kTilesLds = kPart + 4u * NA * 16u * 4u;
  static_assert(2 * kTilesLds <= 160u * 1024u, "two workgroups per CU");
};
template <int B>
constexpr int ring_slots() {
  return B > 4 ? 8 : 4;
}

#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
// 16 (or 4) bytes per lane from global memory into LDS at lds + 16 l (4 l);
// lds must be wave-uniform. m0 is not otherwise used by this kernel; the
// clobber tells the compiler it changes. The _nt forms carry the
// nontemporal hint: the weights are read once per launch, and a stream of
// them without it runs about 10% slower (70B gate/up at 4 rows: 57-59
// against 60-61 us); the activation, read by every workgroup, keeps the
// default policy.
__device__ __forceinline__ void ring_dma16(const uint8_t* src, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off" ::"v"(src), "s"(lds)
               : "memory", "m0");
}
__device__ __forceinline__ void ring_dma16_nt(const uint8_t* src, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off nt" ::"v"(src), "s"(lds)
               : "memory", "m0");
}
__device__ __forceinline__ void ring_dma4(const uint8_t* src, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dword %0, off" ::"v"(src), "s"(lds)
               : "memory", "m0");
}
__device__ __forceinline__ void ring_dma4_nt(const uint8_t* src, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dword %0, off nt" ::"v"(src), "s"(lds)
               : "memory", "m0");
}
#pragma clang diagnostic pop
// s_waitcnt: at most n vector-memory operations of the wave outstanding, and
// all of its LDS operations complete (a barrier after it publishes the
// wave's LDS writes)
constexpr int ring_wait_imm(int n) { return (n & 15) | (((n >> 4) & 3) << 14) | (7 << 4); }

// Direct-load sources of one 16-row tile (first row row0) for this wave: its 4
// weight rows (row r's lane l fetches block l ^ r of each chunk) and 2 x 2
// rows of headers, 4 bytes per lane, row r's 16-B header of super-block sb
// fetched into unit sb ^ ((r >> 1) & 7) of the row's 128 B ((r >> 1) & 7 is
// 2 wv + h for this wave's header rows). Rows past the end repeat the last.
struct RingSrc {
  const uint8_t* w[4];
  const uint8_t* h[2];
};
__device__ __forceinline__ RingSrc ring_tile_src(const GemvArgs& g, int64_t row0, uint32_t lane, uint32_t wv) {
  RingSrc src;
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const uint32_t ri = 4 * wv + r;
    const int64_t row = row0 + ri < g.n ? row0 + ri : g.n - 1;
    src.w[r] = g.w + row * g.row_bytes + g.hdr_bytes + 16u * (lane ^ ri);
  }
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int64_t rr = row0 + 4 * wv + 2 * h + (lane >> 5);
    src.h[h] = g.w + (rr < g.n ? rr : g.n - 1) * g.row_bytes + 16u * (((lane & 31u) >> 2) ^ (2 * wv + h)) +
               4u * (lane & 3u);
  }
  return src;
}
// chunk c of the tile's weights and headers into the stage at LDS address st
__device__ __forceinline__ void ring_issue_weights(const RingSrc& src, uint32_t c, uint32_t st, uint32_t wv) {
#pragma unroll
  for (int r = 0; r < 4; ++r)
    ring_dma16_nt(src.w[r] + 1024u * c, __builtin_amdgcn_readfirstlane(st + (4 * wv + r) * 1024u));
#pragma unroll
  for (int h = 0; h < 2; ++h)
    ring_dma4_nt(src.h[h] + 128u * c, __builtin_amdgcn_readfirstlane(st + kRingW + wv * 512u + h * 256u));
}
// Activation slots 4 t + wv of this wave (t < NA / 4), row min(slot, B - 1):
// codes with 16-B unit U fetched into unit U ^ ((wv & 1) | (wv & 2) << 2) of
// the slot, and (d, sum) pairs.
template <int B>
struct RingAct {
  const uint8_t* a[ring_slots<B>() / 4];
  const uint8_t* d[ring_slots<B>() / 4];
};
template <int B>
__device__ __forceinline__ RingAct<B> ring_act_src(const GemvArgs& g, uint32_t lane, uint32_t wv) {
  RingAct<B> src;
  const uint32_t asw = (wv & 1u) | ((wv & 2u) << 2);
#pragma unroll
  for (int t = 0; t < ring_slots<B>() / 4; ++t) {
    const uint32_t slot = 4u * t + wv;
    const uint32_t arow = slot < static_cast<uint32_t>(B) ? slot : B - 1;
    src.a[t] = g.aq + arow * g.nb * 32u + 16u * (lane ^ asw);
    src.d[t] = g.ads + 8u * (arow * g.nb) + 4u * lane;
  }
  return src;
}
template <int B>
__device__ __forceinline__ void ring_issue_acts(const RingAct<B>& src, uint32_t c, uint32_t st, uint32_t wv) {
  typedef RingLayout<ring_slots<B>()> L;
#pragma unroll
  for (int t = 0; t < ring_slots<B>() / 4; ++t) {
    const uint32_t slot = 4u * t + wv;
#pragma unroll
    for (int h = 0; h < 2; ++h)
      ring_dma16(src.a[t] + 2048u * c + 1024u * h, __builtin_amdgcn_readfirstlane(st + L::kA + slot * 2048u + h * 1024u));
#pragma unroll
    for (int h = 0; h < 2; ++h)
      ring_dma4(src.d[t] + 512u * c + 256u * h, __builtin_amdgcn_readfirstlane(st + L::kD + slot * 512u + h * 256u));
  }
}

// Per-lane LDS read addresses of a stage (relative to the stage).
template <int NG>  // groups of 4 activation rows
struct RingLane {
  uint32_t w_row;             // weight row i's KiB
  uint32_t w_blk;             // 16 wv + q: the lane's block at u = 0 (+ 4 u), XORed with i
  uint32_t i;
  uint32_t a_base[NG][2][2];  // A operand of group G [u & 1][half] (+ 256 (u >> 1)); zero lanes: the zero slots
  uint32_t a_stage[NG];       // stage stride of the A reads (0 for the zero lanes)
  uint32_t h_base[2];         // row i's header of super-block 2 wv + (u >> 1)
  uint32_t d_base;            // (d, sum) of block 16 wv + q of activation row 0 (+ 512 a + 32 u)
  uint32_t q;
};
template <int B>
__device__ __forceinline__ RingLane<ring_slots<B>() / 4> ring_lane(uint32_t lane, uint32_t wv) {
  typedef RingLayout<ring_slots<B>()> Lay;
  RingLane<ring_slots<B>() / 4> L;
  const uint32_t i = lane & 15u, q = lane >> 4;  // weight row (B column), k-group
  const uint32_t aa = lane & 3u, ab = (lane & 15u) >> 2;
  // A operand of group G: activation row 4 G + aa, block 16 wv + 4 u + ab, bytes [16 h, 16 h + 16),
  // unit 32 wv + 8 u + 2 q + h swizzled as the loads placed it; the lanes outside row ab == q of
  // their k-group read zeros, from a slot that the active lanes of that k-group leave free
#pragma unroll
  for (int G = 0; G < ring_slots<B>() / 4; ++G) {
    const bool anz = ab == q && 4u * G + aa < static_cast<uint32_t>(B);
#pragma unroll
    for (int uo = 0; uo < 2; ++uo)
#pragma unroll
      for (int hh = 0; hh < 2; ++hh)
        L.a_base[G][uo][hh] = anz ? Lay::kA + (4u * G + aa) * 2048u +
                                        16u * (32u * wv + 8u * (uo ^ (aa >> 1)) + 2u * q + (hh ^ (aa & 1u)))
                                  : Lay::kZero + 16u * (2u * q + 4u);
    L.a_stage[G] = anz ? Lay::kStage : 0u;
  }
#pragma unroll
  for (int t = 0; t < 2; ++t) L.h_base[t] = kRingW + 128u * i + 16u * ((2u * wv + t) ^ ((i >> 1) & 7u));
  L.d_base = Lay::kD + (16u * wv + q) * 8u;
  L.w_row = i * 1024u;
  L.w_blk = 16u * wv + q;
  L.i = i;
  L.q = q;
  return L;
}

// The stage of parity par: 4 steps of 2 MFMAs per group of 4 activation
// rows, each followed by this lane's scale steps for its (row, block).
template <int B>
__device__ __forceinline__ void ring_chunk(const uint8_t* smem, uint32_t par, const RingLane<ring_slots<B>() / 4>& L,
                                           float (&acc)[B]) {
  constexpr int NG = ring_slots<B>() / 4;
  const uint32_t cur = par * RingLayout<ring_slots<B>()>::kStage;
  typedef int v4i __attribute__((ext_vector_type(4)));
  v4i cinit;
#pragma unroll
  for (int v = 0; v < 4; ++v) cinit[v] = kMagicBits;
  const uint32_t msk = 0x0F0F0F0Fu;
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    const uint32_t b = L.w_blk + 4u * u;  // this lane's block of the chunk
    const uint4 w = *reinterpret_cast<const uint4*>(smem + cur + L.w_row + 16u * (b ^ L.i));
    // the unpack order of dot_nib32: low, then high nibbles of each dword
    v4i w0, w1;
    w0[0] = w.x & msk; w0[1] = (w.x >> 4) & msk; w0[2] = w.y & msk; w0[3] = (w.y >> 4) & msk;
    w1[0] = w.z & msk; w1[1] = (w.z >> 4) & msk; w1[2] = w.w & msk; w1[3] = (w.w >> 4) & msk;
    v4i d[NG];
#pragma unroll
    for (int G = 0; G < NG; ++G) {
      const uint32_t ao = par * L.a_stage[G] + 256u * (u >> 1);
      const v4i a0 = *reinterpret_cast<const v4i*>(smem + L.a_base[G][u & 1][0] + ao);
      const v4i a1 = *reinterpret_cast<const v4i*>(smem + L.a_base[G][u & 1][1] + ao);
      d[G] = __builtin_amdgcn_mfma_i32_16x16x64_i8(a0, w0, cinit, 0, 0, 0);
      d[G] = __builtin_amdgcn_mfma_i32_16x16x64_i8(a1, w1, d[G], 0, 0, 0);  // 1.5 * 2^23 + S per activation row
    }
    const uint4 hd = *reinterpret_cast<const uint4*>(smem + cur + L.h_base[u >> 1]);
    const int j = static_cast<int>((4u * u + L.q) & 7u);
    const float sw = half_bits_to_float(hd.x) * static_cast<float>(q4k_sc(hd, j));
    const float wm = half_bits_to_float(hd.x >> 16) * static_cast<float>(q4k_mn(hd, j));
    const float ncs = -kMagic * sw;
#pragma unroll
    for (int a = 0; a < B; ++a) {
      const float2 ds = *reinterpret_cast<const float2*>(smem + cur + L.d_base + a * 512u + 32u * u);
      const float t = fmaf(__int_as_float(d[a >> 2][a & 3]), sw, ncs);          // S * d * sc_j, exact
      const float t2 = fmaf(wm, static_cast<float>(__float_as_int(ds.y)), t);  // + d_min * mn_j * A
      acc[a] = fmaf(t2, ds.x, acc[a]);
    }
  }
}

// Wave w < ceil(B / 4) adds the 4 waves' partial sums of activation rows 4 w ..
// 4 w + 3, in wave order, and stores them (rows from row0 on).
template <int B>
__device__ __forceinline__ void ring_store(const GemvArgs& g, const float* part, int64_t row0, uint32_t lane,
                                           uint32_t wv) {
  constexpr uint32_t NA = ring_slots<B>();
  const uint32_t a = 4u * wv + (lane >> 4), r = lane & 15u;
  if (a < static_cast<uint32_t>(B)) {
    const float v = ((part[a * 16 + r] + part[(NA + a) * 16 + r]) + part[(2 * NA + a) * 16 + r]) +
                    part[(3 * NA + a) * 16 + r];
    if (row0 + r < g.n) g.y[a * g.ldy + row0 + r] = v;
  }
}

// One 16-row tile (rows 16 tile ...) of the product g.
template <int B, bool SYNC>
__device__ __forceinline__ void ring_one_tile(const GemvArgs& g, int64_t tile) {
  static_assert(B >= 1 && B <= 8, "up to 8 activation rows");
  typedef RingLayout<ring_slots<B>()> Lay;
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
  const uint32_t lane = threadIdx.x & 63u;
  const uint32_t wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int64_t row0 = tile * 16;
  const uint32_t lds0 = static_cast<uint32_t>(reinterpret_cast<uintptr_t>(smem));
  const uint32_t nc = g.nb >> 6;  // the launcher guarantees nb % 64 == 0
  uint64_t tag = 0;
  if constexpr (SYNC) {
    tag = launch_tag();
    produce<B>(g, tag);
  }
  const RingSrc src = ring_tile_src(g, row0, lane, wv);
  const RingAct<B> act = ring_act_src<B>(g, lane, wv);
  for (uint32_t e = threadIdx.x; e < kRingZero / 16; e += 256u)
    *reinterpret_cast<uint4*>(smem + Lay::kZero + 16u * e) = make_uint4(0, 0, 0, 0);
  ring_issue_weights(src, 0, lds0, wv);  // in flight while the activation is awaited
  if constexpr (SYNC) wait_slices<B>(g, tag);
  ring_issue_acts<B>(act, 0, lds0, wv);

  const auto L = ring_lane<B>(lane, wv);
  float acc[B];
#pragma unroll
  for (int a = 0; a < B; ++a) acc[a] = 0.0f;

  for (uint32_t c = 0; c < nc; ++c) {
    __builtin_amdgcn_s_waitcnt(ring_wait_imm(0));  // this wave's loads of stage c are in LDS
    __syncthreads();                               // everyone's; stage c + 1's buffer is free
    if (c + 1 < nc) {
      const uint32_t nxt = lds0 + ((c + 1) & 1u) * Lay::kStage;
      ring_issue_weights(src, c + 1, nxt, wv);
      ring_issue_acts<B>(act, c + 1, nxt, wv);
    }
    ring_chunk<B>(smem, c & 1u, L, acc);
  }
  // the 4 k-groups of a wave, then the 4 waves, in a fixed order
#pragma unroll
  for (int a = 0; a < B; ++a) {
    float v = acc[a];
    v += __shfl_xor(v, 16, 64);
    v += __shfl_xor(v, 32, 64);
    acc[a] = v;
  }
  __builtin_amdgcn_s_waitcnt(ring_wait_imm(0));
  __syncthreads();  // every wave is done with the stages
  float* part = reinterpret_cast<float*>(smem);  // [4 waves][NA][16]
  if (lane < 16) {
#pragma unroll
    for (int a = 0; a < B; ++a) part[(wv * ring_slots<B>() + a) * 16 + lane] = acc[a];
  }
  __builtin_amdgcn_s_waitcnt(ring_wait_imm(0));
  __syncthreads();
  ring_store<B>(g, part, row0, lane, wv);
}

// One 16-row tile per workgroup (grid = tiles).
template <int B, bool SYNC>
__global__ __launch_bounds__(256) void gemv_ring_kernel(GemvArgs g) {
  ring_one_tile<B, SYNC>(g, blockIdx.x);
}

// A fixed grid walking the tiles: workgroup w takes tiles w, w + gridDim.x, ...,
// and the ring runs on across them, so each tile's first chunk is loaded while
// the previous tile's last one is computed. The waves' partial sums of tile j
// go to LDS at the end of its last chunk, and are added and stored after the
// next barrier; a tile has at least two chunks (the launcher), so the next
// tile's sums are written after one more barrier, when those reads are done.
// The sums are the one-tile kernel's, in the same order.
template <int B, bool SYNC>
__global__ __launch_bounds__(256) void gemv_ring_tiles_kernel(GemvArgs g) {
  static_assert(B >= 1 && B <= 8, "up to 8 activation rows");
  typedef RingLayout<ring_slots<B>()> Lay;
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
  const uint32_t lane = threadIdx.x & 63u;
  const uint32_t wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const uint32_t lds0 = static_cast<uint32_t>(reinterpret_cast<uintptr_t>(smem));
  const uint32_t nc = g.nb >> 6;  // the launcher guarantees nb % 64 == 0 and nc >= 2
  const int64_t ntile = (g.n + 15) / 16;
  const uint32_t mytiles = static_cast<uint32_t>((ntile - 1 - blockIdx.x) / gridDim.x + 1);  // grid <= tiles
  const uint32_t total = mytiles * nc;  // stages of this workgroup
  auto tile_row0 = [&](uint32_t j) {
    return (static_cast<int64_t>(blockIdx.x) + static_cast<int64_t>(j) * gridDim.x) * 16;
  };
  uint64_t tag = 0;
  if constexpr (SYNC) {
    tag = launch_tag();
    produce<B>(g, tag);
  }
  RingSrc src = ring_tile_src(g, tile_row0(0), lane, wv);
  const RingAct<B> act = ring_act_src<B>(g, lane, wv);
  for (uint32_t e = threadIdx.x; e < kRingZero / 16; e += 256u)
    *reinterpret_cast<uint4*>(smem + Lay::kZero + 16u * e) = make_uint4(0, 0, 0, 0);
  ring_issue_weights(src, 0, lds0, wv);  // in flight while the activation is awaited
  if constexpr (SYNC) wait_slices<B>(g, tag);
  ring_issue_acts<B>(act, 0, lds0, wv);

  const auto L = ring_lane<B>(lane, wv);
  float acc[B];
#pragma unroll
  for (int a = 0; a < B; ++a) acc[a] = 0.0f;
  float* part = reinterpret_cast<float*>(smem + Lay::kPart);  // [4 waves][NA][16]

  uint32_t j = 0, c = 0;  // tile and chunk of stage s
  for (uint32_t s = 0; s < total; ++s) {
    __builtin_amdgcn_s_waitcnt(ring_wait_imm(0));  // this wave's loads of stage s are in LDS
    __syncthreads();                               // everyone's; stage s + 1's buffer is free
    if (c == 0 && j > 0) ring_store<B>(g, part, tile_row0(j - 1), lane, wv);
    if (s + 1 < total) {
      const uint32_t nxt = lds0 + ((s + 1) & 1u) * Lay::kStage;
      uint32_t cn = c + 1;
      if (cn == nc) {
        cn = 0;
        src = ring_tile_src(g, tile_row0(j + 1), lane, wv);
      }
      ring_issue_weights(src, cn, nxt, wv);
      ring_issue_acts<B>(act, cn, nxt, wv);
    }
    ring_chunk<B>(smem, s & 1u, L, acc);
    if (++c == nc) {
      // the 4 k-groups of a wave, then (in ring_store) the 4 waves, in a fixed order
#pragma unroll
      for (int a = 0; a < B; ++a) {
        float v = acc[a];
        v += __shfl_xor(v, 16, 64);
        v += __shfl_xor(v, 32, 64);
        if (lane < 16) part[(wv * ring_slots<B>() + a) * 16 + lane] = v;
        acc[a] = 0.0f;
      }
      c = 0;
      ++j;
    }
  }
  __builtin_amdgcn_s_waitcnt(ring_wait_imm(0));
  __syncthreads();
  ring_store<B>(g, part, tile_row0(j - 1), lane, wv);
}

// Several independent products in one launch (a descriptor list, e.g. the
// q, k and v matrices of a layer kept as separate buffers): the workgroups
// of descriptor i are [first[i], first[i+1]) and run the classic kernel on
// it. Quantized activations only.
struct GemvMulti {
  GemvArgs d[kGemvMultiMax];
  uint32_t first[kGemvMultiMax + 1];
  int count;
};

// The matrix-core form of the descriptor list (Q4_K, 2-8 rows, every k a
// multiple of 2048): workgroups [first[i], first[i+1]) take the 16-row tiles
// of descriptor i, each computed as the one-tile kernel computes it, so each
// output is qblk_gemv's bit for bit.
template <int B>
__global__ __launch_bounds__(256) void gemv_ring_multi_kernel(GemvMulti m) {
  const uint32_t block = blockIdx.x;
  int i = 0;
#pragma unroll
  for (int t = 1; t < kGemvMultiMax; ++t)
    if (t < m.count && block >= m.first[t]) i = t;  // uniform
  ring_one_tile<B, false>(m.d[i], block - m.first[i]);
}


template <int TYPE, int B, int R, int U, bool ALDS>
__global__ __launch_bounds__(256) void gemv_multi_kernel(GemvMulti m) {
  const uint32_t block = blockIdx.x;
  int i = 0;
#pragma unroll
  for (int t = 1; t < kGemvMultiMax; ++t)
    if (t < m.count && block >= m.first[t]) i = t;  // uniform
  gemv_body<TYPE, B, R, U, false, ALDS>(m.d[i], block - m.first[i]);
}

// Pipelined variant: chunk c+1's weights (and, fused, its fp32 activations)
// are requested before chunk c is computed, so every wave keeps two chunks in
// flight. FUSED: per chunk, the workgroup's 256 threads quantize its 64
// activation blocks (one block per quad of lanes, 8 elements per lane, the
// qblk_quantize_act arithmetic) into one of two LDS slots; one barrier per
// chunk publishes them. B activation rows: B blocks per quad per chunk.
template <int TYPE, int B, int R, bool FUSED, bool SYNC = false, bool ALDS = false>
__global__ __launch_bounds__(256) void gemv_pipe_kernel(GemvArgs g) {
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
  uint8_t* s_codes = smem;                                           // [2][B][64*32]
  float2* s_ds = reinterpret_cast<float2*>(smem + 2 * B * 64 * 32);  // [2][B][64]
  const uint32_t tid = threadIdx.x;
  const uint32_t lane = tid & 63;
  const int64_t wave = static_cast<int64_t>(blockIdx.x) * kWavesPerBlock +
                       __builtin_amdgcn_readfirstlane(static_cast<int>(tid >> 6));
  const int64_t row0 = wave * R;
  uint64_t tag = 0;
  if constexpr (SYNC) {
    tag = launch_tag();
    produce<B>(g, tag);
  }
  if (!FUSED && !SYNC && !ALDS && row0 >= g.n) return;  // whole wave
  const bool active = row0 < g.n;
  const uint32_t nchunks = (g.nb + 63u) >> 6;
  const uint8_t* wrow[R];
#pragma unroll
  for (int r = 0; r < R; ++r) {
    const int64_t rr = row0 + r < g.n ? row0 + r : g.n - 1;
    wrow[r] = g.w + rr * g.row_bytes;
  }

  WChunk<TYPE> wa[R], wb[R];
  WScale<TYPE> sa[R], sb[R];
  float4 xa[B][2], xb[B][2];  // fused: this lane's 8 fp32 elements of each row
  const uint32_t qsub = tid & 3;   // fused: element group inside the block
  const uint32_t qblk = tid >> 2;  // fused: block (0..63) of the chunk

  auto issue = [&](uint32_t c, WChunk<TYPE>(&w)[R], WScale<TYPE>(&s)[R], float4(&xv)[B][2]) {
    const uint32_t blk = (c << 6) + lane;
    if (active && blk < g.nb) {
#pragma unroll
      for (int r = 0; r < R; ++r) load_block<TYPE>(wrow[r], g.hdr_bytes, blk, w[r], s[r]);
    }
    if constexpr (FUSED) {
      const uint32_t qb = (c << 6) + qblk;
      if (qb < g.nb) {
#pragma unroll
        for (int b = 0; b < B; ++b) {
          const float* src = g.x + b * g.ldx + 32u * qb + 8u * qsub;
          xv[b][0] = *reinterpret_cast<const float4*>(src);
          xv[b][1] = *reinterpret_cast<const float4*>(src + 4);
        }
      }
    }
  };

  float acc[R][B];
#pragma unroll
  for (int r = 0; r < R; ++r)
#pragma unroll
    for (int b = 0; b < B; ++b) acc[r][b] = 0.0f;

  auto consume = [&](uint32_t c, const WChunk<TYPE>(&w)[R], const WScale<TYPE>(&s)[R],
                     const float4(&xv)[B][2]) {
    const uint32_t slot = c & 1;
    if constexpr (FUSED) {
      const uint32_t qb = (c << 6) + qblk;
      if (qb < g.nb) {
#pragma unroll
        for (int b = 0; b < B; ++b) {
          const float e[8] = {xv[b][0].x, xv[b][0].y, xv[b][0].z, xv[b][0].w,
                              xv[b][1].x, xv[b][1].y, xv[b][1].z, xv[b][1].w};
          const Q8Group q = quantize_group8(e);
          *reinterpret_cast<uint2*>(s_codes + (slot * B + b) * 2048u + 32u * qblk + 8u * qsub) =
              q.codes;
          if (qsub == 0) s_ds[(slot * B + b) * 64u + qblk] = make_float2(q.d, __int_as_float(q.sum));
        }
      }
      __syncthreads();
    }
    const uint32_t blk = (c << 6) + lane;
    if (!active || blk >= g.nb) return;
    uint4 a[B][1][2];
    float2 ds[B][1];
#pragma unroll
    for (int b = 0; b < B; ++b) {
      if constexpr (FUSED) {
        const uint8_t* ap = s_codes + (slot * B + b) * 2048u + 32u * lane;
        a[b][0][0] = *reinterpret_cast<const uint4*>(ap);
        a[b][0][1] = *reinterpret_cast<const uint4*>(ap + 16);
        ds[b][0] = s_ds[(slot * B + b) * 64u + lane];
      }
    }
    if constexpr (!FUSED) load_act_block<B, 1, ALDS>(g, smem, blk, 0, a, ds);
#pragma unroll
    for (int r = 0; r < R; ++r) block_fma<TYPE, B>(lane, w[r], s[r], a, ds, 0, acc[r]);
  };

  issue(0, wa, sa, xa);
  if constexpr (SYNC || ALDS) {
    // both chunk buffers' weight loads are in flight while the activation
    // is awaited / staged
    if (1 < nchunks) issue(1, wb, sb, xb);
    if constexpr (SYNC) wait_slices<B>(g, tag);
    if constexpr (ALDS) {
      stage_acts<B>(g, smem);
      __syncthreads();
    }
    if (!active) return;
  }
  for (uint32_t c = 0; c < nchunks; c += 2) {
    if (c + 1 < nchunks && !((SYNC || ALDS) && c == 0)) issue(c + 1, wb, sb, xb);
    consume(c, wa, sa, xa);
    if (c + 1 >= nchunks) break;
    if (c + 2 < nchunks) issue(c + 2, wa, sa, xa);
    consume(c + 1, wb, sb, xb);
  }

  if (!active) return;
#pragma unroll
  for (int r = 0; r < R; ++r) {
#pragma unroll
    for (int b = 0; b < B; ++b) {
      const float v = wave_sum_dpp(acc[r][b]);
      if (lane == 63 && row0 + r < g.n) g.y[b * g.ldy + row0 + r] = v;
    }
  }
}

// Everything a launch needs besides the kernel variant.
struct Plan {
  WeightView W;
  int64_t n;
  int64_t nb;
  ActView A;          // quantized activations (for SYNC: the workspace buffer)
  float* y;
  int64_t ldy;
  const float* x;     // fp32 activations (fused variants)
  int64_t ldx;
  GemvWork work;      // SYNC: activation buffer, flags, fallback counter
  int64_t wait_ticks;
};

inline GemvArgs make_args(const Plan& p) {
  GemvArgs g;
  g.x = p.x;
  g.ldx = p.ldx;
  g.w = p.W.base;
  g.row_bytes = p.W.row_bytes;
  g.hdr_bytes = static_cast<uint32_t>(p.W.hdr_bytes);
  g.n = p.n;
  g.nb = static_cast<uint32_t>(p.nb);
  g.aq = p.A.q;
  g.ads = p.A.ds;
  g.y = p.y;
  g.ldy = p.ldy;
  g.xq_codes = p.work.act;
  g.xq_ds = p.work.act ? p.work.act + (p.A.ds - p.A.q) : nullptr;
  g.flags = p.work.flags;
  g.nslices = static_cast<uint32_t>((p.nb + 63) / 64);
  g.flag_stride = static_cast<uint32_t>(gemv_flag_stride(p.nb * 32));
  g.fallbacks = p.work.fallbacks;
  g.wait_ticks = static_cast<uint64_t>(p.wait_ticks);
  return g;
}

template <int R>
inline dim3 grid_for(int64_t n) {
  const int64_t waves = (n + R - 1) / R;
  return dim3(static_cast<uint32_t>((waves + kWavesPerBlock - 1) / kWavesPerBlock));
}

// The activation rows are staged in LDS when they fit the limit for their count.
inline bool stage_in_lds(int b, int64_t nb) { return gemv_stage_acts_in_lds(b, nb); }

template <int TYPE, int B, int R, bool FUSED, bool SYNC>
hipError_t launch_pipe(const Plan& p, hipStream_t s) {
  if (!FUSED && stage_in_lds(B, p.nb)) {
    hipLaunchKernelGGL((gemv_pipe_kernel<TYPE, B, R, false, SYNC, true>), grid_for<R>(p.n),
                       dim3(64 * kWavesPerBlock), act_lds_bytes(B, static_cast<uint32_t>(p.nb)),
                       s, make_args(p));
  } else {
    const size_t shmem = FUSED ? static_cast<size_t>(2 * B * 64 * 40) : 0;
    hipLaunchKernelGGL((gemv_pipe_kernel<TYPE, B, R, FUSED, SYNC, false>), grid_for<R>(p.n),
                       dim3(64 * kWavesPerBlock), shmem, s, make_args(p));
  }
  return hipGetLastError();
}

template <int TYPE, int B, int R, int U, bool SYNC, int WAVES = kWavesPerBlock>
hipError_t launch_cfg(const Plan& p, hipStream_t s) {
  const dim3 grid(static_cast<uint32_t>(((p.n + R - 1) / R + WAVES - 1) / WAVES));
  if (stage_in_lds(B, p.nb)) {
    hipLaunchKernelGGL((gemv_kernel<TYPE, B, R, U, SYNC, true, WAVES>), grid, dim3(64 * WAVES),
                       act_lds_bytes(B, static_cast<uint32_t>(p.nb)), s, make_args(p));
  } else {
    hipLaunchKernelGGL((gemv_kernel<TYPE, B, R, U, SYNC, false, WAVES>), grid, dim3(64 * WAVES), 0, s,
                       make_args(p));
  }
  return hipGetLastError();
}

// The matrix-core kernels (Q4_K, 2-8 rows, k a multiple of 2048; select_gemv
// only picks them there): one 16-row tile per workgroup, or the tile-walking
// grid (k at least 4096: two chunks per tile).
template <int TYPE, int B, bool SYNC>
hipError_t launch_ring(const Plan& p, bool tiles_grid, hipStream_t s) {
  if constexpr (TYPE == kQ4_K && B >= 2 && B <= 8) {
    typedef RingLayout<ring_slots<B>()> Lay;
    if (p.nb % 64 != 0) return hipErrorInvalidValue;
    if (tiles_grid) {
      if (p.nb < 128) return hipErrorInvalidValue;
      hipLaunchKernelGGL((gemv_ring_tiles_kernel<B, SYNC>), dim3(static_cast<uint32_t>(kRingGrid)), dim3(256),
                         Lay::kTilesLds, s, make_args(p));
    } else {
      hipLaunchKernelGGL((gemv_ring_kernel<B, SYNC>), dim3(static_cast<uint32_t>((p.n + 15) / 16)), dim3(256),
                         Lay::kLds, s, make_args(p));
    }
    return hipGetLastError();
  } else {
    return hipErrorInvalidValue;
  }
}

// How the activation reaches the kernel.
enum Mode { kQuantized = kGemvQuantized, kLdsFused = kGemvLdsFused, kInLaunch = kGemvInLaunch };

template <int TYPE, int B, int MODE>
hipError_t launch_b(const Plan& p, hipStream_t s) {
  constexpr bool SYNC = MODE == kInLaunch;
  const GemvVariant v = select_gemv(TYPE, p.n, p.nb * 32, B, MODE);
  const int ru = 10 * v.r + v.u;
  if constexpr (MODE == kLdsFused) {
    if (v.r == 4) return launch_pipe<TYPE, B, 4, true, false>(p, s);
    return launch_pipe<TYPE, B, 2, true, false>(p, s);
  } else if constexpr (B == 1) {
    switch (ru) {
      case 41: return launch_cfg<TYPE, 1, 4, 1, SYNC>(p, s);
      case 22: return launch_cfg<TYPE, 1, 2, 2, SYNC>(p, s);
      case 21: return launch_cfg<TYPE, 1, 2, 1, SYNC>(p, s);
      case 12: return launch_cfg<TYPE, 1, 1, 2, SYNC>(p, s);
      default: return hipErrorInvalidValue;
    }
  } else {
    if (v.ring) return launch_ring<TYPE, B, SYNC>(p, v.ring_tiles, s);
    if (v.waves == 8) {
      if (ru == 81) return launch_cfg<TYPE, B, 8, 1, SYNC, 8>(p, s);
      if (ru == 41) return launch_cfg<TYPE, B, 4, 1, SYNC, 8>(p, s);
      return hipErrorInvalidValue;
    }
    switch (ru) {
      case 81: return launch_cfg<TYPE, B, 8, 1, SYNC>(p, s);
      case 41: return launch_cfg<TYPE, B, 4, 1, SYNC>(p, s);
      case 21: return launch_cfg<TYPE, B, 2, 1, SYNC>(p, s);
      case 11: return launch_cfg<TYPE, B, 1, 1, SYNC>(p, s);
      default: return hipErrorInvalidValue;
    }
  }
}

template <int TYPE, int MODE = kQuantized>
hipError_t launch_batch(int b, const Plan& p, hipStream_t s) {
  switch (b) {
    case 1: return launch_b<TYPE, 1, MODE>(p, s);
    case 2: return launch_b<TYPE, 2, MODE>(p, s);
    case 3: return launch_b<TYPE, 3, MODE>(p, s);
    case 4: return launch_b<TYPE, 4, MODE>(p, s);
    case 5: return launch_b<TYPE, 5, MODE>(p, s);
    case 6: return launch_b<TYPE, 6, MODE>(p, s);
    case 7: return launch_b<TYPE, 7, MODE>(p, s);
    default: return launch_b<TYPE, 8, MODE>(p, s);
  }
}

template <int MODE>
hipError_t launch_type(int type, int b, const Plan& p, hipStream_t s) {
  switch (type) {
    case kQ4_0: return launch_batch<kQ4_0, MODE>(b, p, s);
    case kQ8_0: return launch_batch<kQ8_0, MODE>(b, p, s);
    case kQ4_0H: return launch_batch<kQ4_0H, MODE>(b, p, s);
    default: return launch_batch<kQ4_K, MODE>(b, p, s);
  }
}

}  // namespace

hipError_t launch_gemv(int type, const void* wq, int64_t n, int64_t k, const void* xq,
                       int64_t batch, float* y, int64_t ldy, hipStream_t s) {
  Plan p{};
  p.W.base = static_cast<const uint8_t*>(wq);
  p.W.row_bytes = row_bytes(type, k);
  p.W.hdr_bytes = header_bytes(type, k);
  p.n = n;
  p.nb = k / 32;
  p.ldy = ldy;
  const ActView full = make_act(xq, batch, k);
  // up to 8 activation rows per launch; the weights are re-streamed for each
  // group of 8 (large batches belong to qblk_gemm)
  for (int64_t b0 = 0; b0 < batch; b0 += 8) {
    const int bc = static_cast<int>(batch - b0 < 8 ? batch - b0 : 8);
    p.A = full;
    p.A.q = full.q + b0 * k;
    p.A.ds = full.ds + 8 * b0 * p.nb;
    p.y = y + b0 * ldy;
    const hipError_t e = launch_type<kQuantized>(type, bc, p, s);
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

namespace {

template <int TYPE, int B, int R, int U>
hipError_t launch_multi_r(GemvMulti& m, const int64_t* rows, int count, int64_t max_nb, hipStream_t s) {
  uint32_t blocks = 0;
  for (int i = 0; i < count; ++i) {
    m.first[i] = blocks;
    blocks += grid_for<R>(rows[i]).x;
  }
  for (int i = count; i <= kGemvMultiMax; ++i) m.first[i] = blocks;
  m.count = count;
  if (blocks == 0) return hipSuccess;
  if (stage_in_lds(B, max_nb)) {
    hipLaunchKernelGGL((gemv_multi_kernel<TYPE, B, R, U, true>), dim3(blocks), dim3(64 * kWavesPerBlock),
                       act_lds_bytes(B, static_cast<uint32_t>(max_nb)), s, m);
  } else {
    hipLaunchKernelGGL((gemv_multi_kernel<TYPE, B, R, U, false>), dim3(blocks), dim3(64 * kWavesPerBlock), 0, s,
                       m);
  }
  return hipGetLastError();
}

// rows per wave as for the mid-size single products: 2 at batch 1, 4 above
template <int TYPE>
hipError_t launch_multi_type(int b, GemvMulti& m, const int64_t* rows, int count, int64_t max_nb,
                             hipStream_t s) {
  switch (b) {
    case 1: return launch_multi_r<TYPE, 1, 2, 1>(m, rows, count, max_nb, s);
    case 2: return launch_multi_r<TYPE, 2, 4, 1>(m, rows, count, max_nb, s);
    case 3: return launch_multi_r<TYPE, 3, 4, 1>(m, rows, count, max_nb, s);
    case 4: return launch_multi_r<TYPE, 4, 4, 1>(m, rows, count, max_nb, s);
    case 5: return launch_multi_r<TYPE, 5, 4, 1>(m, rows, count, max_nb, s);
    case 6: return launch_multi_r<TYPE, 6, 4, 1>(m, rows, count, max_nb, s);
    case 7: return launch_multi_r<TYPE, 7, 4, 1>(m, rows, count, max_nb, s);
    default: return launch_multi_r<TYPE, 8, 4, 1>(m, rows, count, max_nb, s);
  }
}

}  // namespace

template <int B>
hipError_t launch_ring_multi_b(const GemvMulti& m, hipStream_t s) {
  hipLaunchKernelGGL((gemv_ring_multi_kernel<B>), dim3(m.first[m.count]), dim3(256),
                     RingLayout<ring_slots<B>()>::kLds, s, m);
  return hipGetLastError();
}
hipError_t launch_ring_multi(int b, const GemvMulti& m, hipStream_t s) {
  switch (b) {
    case 2: return launch_ring_multi_b<2>(m, s);
    case 3: return launch_ring_multi_b<3>(m, s);
    case 4: return launch_ring_multi_b<4>(m, s);
    case 5: return launch_ring_multi_b<5>(m, s);
    case 6: return launch_ring_multi_b<6>(m, s);
    case 7: return launch_ring_multi_b<7>(m, s);
    case 8: return launch_ring_multi_b<8>(m, s);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_gemv_multi(int type, const GemvDesc* d, int count, int64_t batch, hipStream_t s) {
  for (int64_t b0 = 0; b0 < batch; b0 += 8) {
    const int bc = static_cast<int>(batch - b0 < 8 ? batch - b0 : 8);
    GemvMulti m{};
    int64_t rows[kGemvMultiMax];
    int used = 0;
    int64_t max_nb = 0;
    for (int i = 0; i < count; ++i) {
      if (d[i].n == 0) continue;
      Plan p{};
      p.W.base = static_cast<const uint8_t*>(d[i].wq);
      p.W.row_bytes = row_bytes(type, d[i].k);
      p.W.hdr_bytes = header_bytes(type, d[i].k);
      p.n = d[i].n;
      p.nb = d[i].k / 32;
      const ActView full = make_act(d[i].xq, batch, d[i].k);
      p.A = full;
      p.A.q = full.q + b0 * d[i].k;
      p.A.ds = full.ds + 8 * b0 * p.nb;
      p.y = d[i].y + b0 * d[i].ldy;
      p.ldy = d[i].ldy;
      m.d[used] = make_args(p);
      rows[used] = p.n;
      max_nb = p.nb > max_nb ? p.nb : max_nb;
      ++used;
    }
    if (used == 0) return hipSuccess;
    hipError_t e;
    bool ring = type == kQ4_K && bc >= 2;
    for (int i = 0; i < used; ++i) ring = ring && m.d[i].nb % 64 == 0;
    if (ring) {
      m.count = used;
      m.first[0] = 0;
      for (int i = 0; i < used; ++i) m.first[i + 1] = m.first[i] + static_cast<uint32_t>((rows[i] + 15) / 16);
      e = launch_ring_multi(bc, m, s);
      if (e != hipSuccess) return e;
      continue;
    }
    switch (type) {
      case kQ4_0: e = launch_multi_type<kQ4_0>(bc, m, rows, used, max_nb, s); break;
      case kQ8_0: e = launch_multi_type<kQ8_0>(bc, m, rows, used, max_nb, s); break;
      case kQ4_0H: e = launch_multi_type<kQ4_0H>(bc, m, rows, used, max_nb, s); break;
      default: e = launch_multi_type<kQ4_K>(bc, m, rows, used, max_nb, s); break;
    }
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

// Fused quantize + GEMV (fp32 activations, batch <= gemv_f32_max_batch(k)):
// one launch streams the weights once. Small single-row products with short
// rows: every workgroup quantizes the activation into its local memory.
// Otherwise the first workgroups quantize it once into the workspace and the
// others wait for it behind their first weight loads (repeating the
// quantization in every workgroup would cost more than the weight stream).
hipError_t launch_gemv_f32(int type, const void* wq, int64_t n, int64_t k, const float* x,
                           int64_t ldx, int64_t batch, float* y, int64_t ldy, const GemvWork& work,
                           int64_t wait_ticks, hipStream_t s) {
  Plan p{};
  p.W.base = static_cast<const uint8_t*>(wq);
  p.W.row_bytes = row_bytes(type, k);
  p.W.hdr_bytes = header_bytes(type, k);
  p.n = n;
  p.nb = k / 32;
  p.y = y;
  p.ldy = ldy;
  p.x = x;
  p.ldx = ldx;
  const int bc = static_cast<int>(batch);
  if (gemv_f32_lds_fused(n, k, batch)) {
    p.A = make_act(nullptr, 0, k);
    return launch_type<kLdsFused>(type, bc, p, s);
  }
  p.A = make_act(work.act, batch, k);
  p.work = work;
  p.wait_ticks = wait_ticks;
  return launch_type<kInLaunch>(type, bc, p, s);
}

// ---------------------------------------------------------------- fixed workspace
// The allocation-free entry point's workspace (qblk_gemv_f32_noalloc): a
// file-scope device array, zero when the code object is loaded. Each GPU the
// library runs on holds its own copy until the process ends. In host code
// `scratch` names a host-side stand-in, never the device memory: kernels get
// the address from hipGetSymbolAddress, looked up once per device.
static __device__ __align__(256) uint8_t scratch[kScratchBytes];

namespace {
constexpr int kMaxScratchDevices = 64;
std::atomic<uint8_t*> g_scratch_addr[kMaxScratchDevices];
}  // namespace

hipError_t gemv_scratch_work(hipStream_t stream, GemvWork* w) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxScratchDevices) return hipErrorInvalidDevice;
  if (stream != nullptr) {
    hipDevice_t sd = 0;
    e = hipStreamGetDevice(stream, &sd);
    if (e != hipSuccess) return e;
    if (static_cast<int>(sd) != dev) return hipErrorInvalidDevice;
  }
  uint8_t* base = g_scratch_addr[dev].load(std::memory_order_acquire);
  if (base == nullptr) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    base = static_cast<uint8_t*>(p);
    g_scratch_addr[dev].store(base, std::memory_order_release);
  }
  w->flags = reinterpret_cast<uint64_t*>(base);
  w->fallbacks = reinterpret_cast<uint32_t*>(base + kScratchFlagBytes - 256);
  w->act = base + kScratchFlagBytes;
  return hipSuccess;
}

}  // namespace qblk
