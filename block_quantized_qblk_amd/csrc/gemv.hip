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
  const uint8_t* aq;   // activation codes [B][k]
  const uint8_t* ads;  // activation (d, sum) [B][nb]
  float* y;
  int64_t ldy;
};

template <int TYPE, int B, int R, int U>
__global__ __launch_bounds__(256) void gemv_kernel(GemvArgs g) {
  const uint32_t lane = threadIdx.x & 63;
  const int64_t wave = static_cast<int64_t>(blockIdx.x) * kWavesPerBlock +
                       __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x >> 6));
  const int64_t row0 = wave * R;
  if (row0 >= g.n) return;  // whole wave
  const uint8_t* wrow[R];
#pragma unroll
  for (int r = 0; r < R; ++r) wrow[r] = g.w + (row0 + r < g.n ? row0 + r : g.n - 1) * g.row_bytes;
  const uint32_t k = g.nb * 32u;

  float acc[R][B];
#pragma unroll
  for (int r = 0; r < R; ++r)
#pragma unroll
    for (int b = 0; b < B; ++b) acc[r][b] = 0.0f;

  const uint32_t nchunks = (g.nb + 63u) >> 6;
  for (uint32_t c0 = 0; c0 < nchunks; c0 += U) {
    WChunk<TYPE> w[R][U];
    WScale<TYPE> s[R][U];
    uint4 a[B][U][2];
    float2 ds[B][U];
    // ---- issue every load of U chunks first
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
    // ---- then the arithmetic
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const uint32_t blk = ((c0 + u) << 6) + lane;
      if (blk >= g.nb) continue;
      const int j = static_cast<int>(lane & 7);  // sub-block inside a Q4_K super-block
#pragma unroll
      for (int r = 0; r < R; ++r) {
        if constexpr (TYPE == kQ4_K) {
          const uint4 h = s[r][u].h;
          const float sw = half_bits_to_float(h.x) * static_cast<float>(q4k_sc(h, j));
          const float wm = half_bits_to_float(h.x >> 16) * static_cast<float>(q4k_mn(h, j));
#pragma unroll
          for (int b = 0; b < B; ++b) {
            const int S = dot_nib32(w[r][u].q, a[b][u][0], a[b][u][1], 0);
            const float asum = static_cast<float>(__float_as_int(ds[b][u].y));
            acc[r][b] = fmaf(ds[b][u].x, fmaf(sw, static_cast<float>(S), wm * asum), acc[r][b]);
          }
        } else if constexpr (TYPE == kQ4_0) {
#pragma unroll
          for (int b = 0; b < B; ++b) {
            const int S = dot_nib32(w[r][u].q, a[b][u][0], a[b][u][1], 0) -
                          8 * __float_as_int(ds[b][u].y);
            acc[r][b] = fmaf(s[r][u].d * ds[b][u].x, static_cast<float>(S), acc[r][b]);
          }
        } else {
#pragma unroll
          for (int b = 0; b < B; ++b) {
            const int S = dot_i8x32(w[r][u].q0, w[r][u].q1, a[b][u][0], a[b][u][1], 0);
            acc[r][b] = fmaf(s[r][u].d * ds[b][u].x, static_cast<float>(S), acc[r][b]);
          }
        }
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

template <int TYPE, int B, int R, int U>
hipError_t launch_cfg(WeightView W, int64_t n, int64_t nb, ActView A, float* y, int64_t ldy,
                      hipStream_t s) {
  const int64_t waves = (n + R - 1) / R;
  const int64_t grid = (waves + kWavesPerBlock - 1) / kWavesPerBlock;
  GemvArgs g;
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

// Rows per wave R and chunks in flight U, from measurements on MI355X: large
// matrices stream best with 4 rows per wave (activation registers reused 4x),
// mid-size ones with 2, small ones (few waves) with 1 row and 2 chunks.
template <int TYPE, int B>
hipError_t launch_b(WeightView W, int64_t n, int64_t nb, ActView A, float* y, int64_t ldy,
                    hipStream_t s) {
  if constexpr (B == 1) {
    if (n >= 8192) return launch_cfg<TYPE, 1, 4, 1>(W, n, nb, A, y, ldy, s);
    if (n >= 3072) return launch_cfg<TYPE, 1, 2, 1>(W, n, nb, A, y, ldy, s);
    return launch_cfg<TYPE, 1, 1, 2>(W, n, nb, A, y, ldy, s);
  } else {
    if (n >= 3072) return launch_cfg<TYPE, B, 2, 1>(W, n, nb, A, y, ldy, s);
    return launch_cfg<TYPE, B, 1, 1>(W, n, nb, A, y, ldy, s);
  }
}

template <int TYPE>
hipError_t launch_batch(int b, WeightView W, int64_t n, int64_t nb, ActView A, float* y,
                        int64_t ldy, hipStream_t s) {
  switch (b) {
    case 1: return launch_b<TYPE, 1>(W, n, nb, A, y, ldy, s);
    case 2: return launch_b<TYPE, 2>(W, n, nb, A, y, ldy, s);
    case 3: return launch_b<TYPE, 3>(W, n, nb, A, y, ldy, s);
    case 4: return launch_b<TYPE, 4>(W, n, nb, A, y, ldy, s);
    case 5: return launch_b<TYPE, 5>(W, n, nb, A, y, ldy, s);
    case 6: return launch_b<TYPE, 6>(W, n, nb, A, y, ldy, s);
    case 7: return launch_b<TYPE, 7>(W, n, nb, A, y, ldy, s);
    default: return launch_b<TYPE, 8>(W, n, nb, A, y, ldy, s);
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
