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

template <int TYPE>
struct WScale;  // one lane's block scale data
template <>
struct WScale<kQ4_0> { float d; };
template <>
struct WScale<kQ8_0> { float d; };
template <>
struct WScale<kQ4_K> { uint4 h; };

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
};

// The per-block arithmetic of one weight row against B activation rows, in
// one fixed order for every kernel variant (so that all variants, fused or
// not, produce bit-identical results): integer dot of the 32 codes, then the
// fp32 scale FMAs, accumulated per lane in ascending block order.
template <int TYPE, int B, int U>
__device__ __forceinline__ void block_fma(uint32_t lane, const WChunk<TYPE>& w,
                                          const WScale<TYPE>& s, const uint4 (&a)[B][U][2],
                                          const float2 (&ds)[B][U], int u, float (&acc)[B]) {
  if constexpr (TYPE == kQ4_K) {
    const int j = static_cast<int>(lane & 7);  // sub-block inside the super-block
    const float sw = half_bits_to_float(s.h.x) * static_cast<float>(q4k_sc(s.h, j));
    const float wm = half_bits_to_float(s.h.x >> 16) * static_cast<float>(q4k_mn(s.h, j));
#pragma unroll
    for (int b = 0; b < B; ++b) {
      const int S = dot_nib32(w.q, a[b][u][0], a[b][u][1], 0);
      const float asum = static_cast<float>(__float_as_int(ds[b][u].y));
      acc[b] = fmaf(ds[b][u].x, fmaf(sw, static_cast<float>(S), wm * asum), acc[b]);
    }
  } else if constexpr (TYPE == kQ4_0) {
#pragma unroll
    for (int b = 0; b < B; ++b) {
      const int S = dot_nib32(w.q, a[b][u][0], a[b][u][1], 0) - 8 * __float_as_int(ds[b][u].y);
      acc[b] = fmaf(s.d * ds[b][u].x, static_cast<float>(S), acc[b]);
    }
  } else {
#pragma unroll
    for (int b = 0; b < B; ++b) {
      const int S = dot_i8x32(w.q0, w.q1, a[b][u][0], a[b][u][1], 0);
      acc[b] = fmaf(s.d * ds[b][u].x, static_cast<float>(S), acc[b]);
    }
  }
}

// Classic variant: each wave issues the loads of U chunks for its R rows,
// then computes them; occupancy hides the latency. Best for large matrices.
template <int TYPE, int B, int R, int U>
__global__ __launch_bounds__(256) void gemv_kernel(GemvArgs g) {
  const uint32_t lane = threadIdx.x & 63;
  const int64_t wave = static_cast<int64_t>(blockIdx.x) * kWavesPerBlock +
                       __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x >> 6));
  const int64_t row0 = wave * R;
  if (row0 >= g.n) return;  // whole wave
  const uint8_t* wrow[R];
#pragma unroll
  for (int r = 0; r < R; ++r) {
    const int64_t rr = row0 + r < g.n ? row0 + r : g.n - 1;
    wrow[r] = g.w + rr * g.row_bytes;
  }
  const uint32_t k = g.nb * 32u;
  const uint32_t nchunks = (g.nb + 63u) >> 6;

  float acc[R][B];
#pragma unroll
  for (int r = 0; r < R; ++r)
#pragma unroll
    for (int b = 0; b < B; ++b) acc[r][b] = 0.0f;

  for (uint32_t c0 = 0; c0 < nchunks; c0 += U) {
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
#pragma unroll
        for (int b = 0; b < B; ++b) {
          const uint8_t* ap = g.aq + b * k;
          a[b][u][0] = load16(ap + 32u * blk);
          a[b][u][1] = load16(ap + (32u * blk + 16u));
          ds[b][u] = *reinterpret_cast<const float2*>(g.ads + 8u * (b * g.nb) + 8u * blk);
        }
      }
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const uint32_t blk = ((c0 + u) << 6) + lane;
      if (blk < g.nb) {
#pragma unroll
        for (int r = 0; r < R; ++r) block_fma<TYPE, B>(lane, w[r][u], s[r][u], a, ds, u, acc[r]);
      }
    }
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

// Pipelined variant: chunk c+1's weights (and, fused, its fp32 activations)
// are requested before chunk c is computed, so every wave keeps two chunks in
// flight. FUSED: per chunk, the workgroup's 256 threads quantize its 64
// activation blocks (one block per quad of lanes, 8 elements per lane, the
// qblk_quantize_act arithmetic) into one of two LDS slots; one barrier per
// chunk publishes them. B activation rows: B blocks per quad per chunk.
template <int TYPE, int B, int R, bool FUSED>
__global__ __launch_bounds__(256) void gemv_pipe_kernel(GemvArgs g) {
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
  uint8_t* s_codes = smem;                                           // [2][B][64*32]
  float2* s_ds = reinterpret_cast<float2*>(smem + 2 * B * 64 * 32);  // [2][B][64]
  const uint32_t tid = threadIdx.x;
  const uint32_t lane = tid & 63;
  const int64_t wave = static_cast<int64_t>(blockIdx.x) * kWavesPerBlock +
                       __builtin_amdgcn_readfirstlane(static_cast<int>(tid >> 6));
  const int64_t row0 = wave * R;
  if (!FUSED && row0 >= g.n) return;  // whole wave
  const bool active = row0 < g.n;
  const uint32_t k = g.nb * 32u;
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
      } else {
        const uint8_t* ap = g.aq + b * k;
        a[b][0][0] = load16(ap + 32u * blk);
        a[b][0][1] = load16(ap + (32u * blk + 16u));
        ds[b][0] = *reinterpret_cast<const float2*>(g.ads + 8u * (b * g.nb) + 8u * blk);
      }
    }
#pragma unroll
    for (int r = 0; r < R; ++r) block_fma<TYPE, B>(lane, w[r], s[r], a, ds, 0, acc[r]);
  };

  issue(0, wa, sa, xa);
  for (uint32_t c = 0; c < nchunks; c += 2) {
    if (c + 1 < nchunks) issue(c + 1, wb, sb, xb);
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

template <int TYPE, int B, int R, bool FUSED>
hipError_t launch_pipe(WeightView W, int64_t n, int64_t nb, ActView A, float* y, int64_t ldy,
                       hipStream_t s, const float* x = nullptr, int64_t ldx = 0) {
  const int64_t waves = (n + R - 1) / R;
  const int64_t grid = (waves + kWavesPerBlock - 1) / kWavesPerBlock;
  GemvArgs g;
  g.x = x;
  g.ldx = ldx;
  g.w = W.base;
  g.row_bytes = W.row_bytes;
  g.hdr_bytes = static_cast<uint32_t>(W.hdr_bytes);
  g.n = n;
  g.nb = static_cast<uint32_t>(nb);
  g.aq = A.q;
  g.ads = A.ds;
  g.y = y;
  g.ldy = ldy;
  const size_t shmem = FUSED ? static_cast<size_t>(2 * B * 64 * 40) : 0;
  hipLaunchKernelGGL((gemv_pipe_kernel<TYPE, B, R, FUSED>), dim3(static_cast<uint32_t>(grid)),
                     dim3(64 * kWavesPerBlock), shmem, s, g);
  return hipGetLastError();
}

template <int TYPE, int B, int R, int U>
hipError_t launch_cfg(WeightView W, int64_t n, int64_t nb, ActView A, float* y, int64_t ldy,
                      hipStream_t s) {
  const int64_t waves = (n + R - 1) / R;
  const int64_t grid = (waves + kWavesPerBlock - 1) / kWavesPerBlock;
  GemvArgs g;
  g.x = nullptr;
  g.ldx = 0;
  g.w = W.base;
  g.row_bytes = W.row_bytes;
  g.hdr_bytes = static_cast<uint32_t>(W.hdr_bytes);
  g.n = n;
  g.nb = static_cast<uint32_t>(nb);
  g.aq = A.q;
  g.ads = A.ds;
  g.y = y;
  g.ldy = ldy;
  hipLaunchKernelGGL((gemv_kernel<TYPE, B, R, U>), dim3(static_cast<uint32_t>(grid)),
                     dim3(64 * kWavesPerBlock), 0, s, g);
  return hipGetLastError();
}

// Kernel variant per shape, from kernel-trace measurements on MI355X over the
// 7B- and 70B-shaped Q4_K matrices (batch 1): the classic kernel with 4 rows
// per wave streams the largest matrices best (6.0-6.3 TB/s), the pipelined
// kernel with 2 rows per wave the mid-size ones, 1 row per wave with 2 chunks
// in flight the small ones. All variants give bit-identical results.
template <int TYPE, int B, bool FUSED = false>
hipError_t launch_b(WeightView W, int64_t n, int64_t nb, ActView A, float* y, int64_t ldy,
                    hipStream_t s, const float* x = nullptr, int64_t ldx = 0) {
  const int64_t k = nb * 32;
  if constexpr (FUSED) {
    if (n >= 8192) return launch_pipe<TYPE, B, 4, true>(W, n, nb, A, y, ldy, s, x, ldx);
    return launch_pipe<TYPE, B, 2, true>(W, n, nb, A, y, ldy, s, x, ldx);
  } else if constexpr (B == 1) {
    if (n >= 16384) {
      if (k >= 8192) return launch_cfg<TYPE, 1, 4, 1>(W, n, nb, A, y, ldy, s);
      return launch_cfg<TYPE, 1, 2, 1>(W, n, nb, A, y, ldy, s);
    }
    if (n >= 8192 && k >= 16384) return launch_cfg<TYPE, 1, 4, 1>(W, n, nb, A, y, ldy, s);
    if (n >= 3072) return launch_pipe<TYPE, 1, 2, false>(W, n, nb, A, y, ldy, s);
    return launch_cfg<TYPE, 1, 1, 2>(W, n, nb, A, y, ldy, s);
  } else {
    if (n >= 3072) return launch_cfg<TYPE, B, 2, 1>(W, n, nb, A, y, ldy, s);
    return launch_cfg<TYPE, B, 1, 1>(W, n, nb, A, y, ldy, s);
  }
}

template <int TYPE, bool FUSED = false>
hipError_t launch_batch(int b, WeightView W, int64_t n, int64_t nb, ActView A, float* y,
                        int64_t ldy, hipStream_t s, const float* x = nullptr, int64_t ldx = 0) {
  switch (b) {
    case 1: return launch_b<TYPE, 1, FUSED>(W, n, nb, A, y, ldy, s, x, ldx);
    case 2: return launch_b<TYPE, 2, FUSED>(W, n, nb, A, y, ldy, s, x, ldx);
    case 3: return launch_b<TYPE, 3, FUSED>(W, n, nb, A, y, ldy, s, x, ldx);
    case 4: return launch_b<TYPE, 4, FUSED>(W, n, nb, A, y, ldy, s, x, ldx);
    case 5: return launch_b<TYPE, 5, FUSED>(W, n, nb, A, y, ldy, s, x, ldx);
    case 6: return launch_b<TYPE, 6, FUSED>(W, n, nb, A, y, ldy, s, x, ldx);
    case 7: return launch_b<TYPE, 7, FUSED>(W, n, nb, A, y, ldy, s, x, ldx);
    default: return launch_b<TYPE, 8, FUSED>(W, n, nb, A, y, ldy, s, x, ldx);
  }
}

}  // namespace

hipError_t launch_gemv(int type, const void* wq, int64_t n, int64_t k, const void* xq,
                       int64_t batch, float* y, int64_t ldy, hipStream_t s) {
  WeightView W;
  W.base = static_cast<const uint8_t*>(wq);
  W.row_bytes = row_bytes(type, k);
  W.hdr_bytes = header_bytes(type, k);
  const ActView full = make_act(xq, batch, k);
  const int64_t nb = k / 32;
  // up to 8 activation rows per launch; the weights are re-streamed for each
  // group of 8 (large batches belong to qblk_gemm)
  for (int64_t b0 = 0; b0 < batch; b0 += 8) {
    const int bc = static_cast<int>(batch - b0 < 8 ? batch - b0 : 8);
    ActView A = full;
    A.q = full.q + b0 * k;
    A.ds = full.ds + 8 * b0 * nb;
    float* yb = y + b0 * ldy;
    hipError_t e;
    switch (type) {
      case kQ4_0: e = launch_batch<kQ4_0>(bc, W, n, nb, A, yb, ldy, s); break;
      case kQ8_0: e = launch_batch<kQ8_0>(bc, W, n, nb, A, yb, ldy, s); break;
      default: e = launch_batch<kQ4_K>(bc, W, n, nb, A, yb, ldy, s); break;
    }
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace qblk

namespace qblk {

// Fused quantize + GEMV: fp32 activations in; the caller guarantees that
// batch <= gemv_f32_max_batch(k), so one launch streams the weights once.
hipError_t launch_gemv_f32(int type, const void* wq, int64_t n, int64_t k, const float* x,
                           int64_t ldx, int64_t batch, float* y, int64_t ldy, hipStream_t s) {
  WeightView W;
  W.base = static_cast<const uint8_t*>(wq);
  W.row_bytes = row_bytes(type, k);
  W.hdr_bytes = header_bytes(type, k);
  const int64_t nb = k / 32;
  const ActView none = make_act(nullptr, 0, k);
  const int bc = static_cast<int>(batch);
  switch (type) {
    case kQ4_0: return launch_batch<kQ4_0, true>(bc, W, n, nb, none, y, ldy, s, x, ldx);
    case kQ8_0: return launch_batch<kQ8_0, true>(bc, W, n, nb, none, y, ldy, s, x, ldx);
    default: return launch_batch<kQ4_K, true>(bc, W, n, nb, none, y, ldy, s, x, ldx);
  }
}

}  // namespace qblk
