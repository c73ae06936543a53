// Prefill-path product Y[m][n] = X * W^T with int8 matrix-core tiles.
//
// Dequantize-free: each 32-block's integer dot product is one
// v_mfma_i32_32x32x32_i8 over a 32x32 output tile (K = 32 is exactly one
// block), and the block scales are applied to the int32 tile in fp32 right
// after it ("llama.cpp 推理引擎", §6.4: scales outside the integer values;
// §5.5 Q4_K sub-block scale and min; §7.3: prefill is compute-bound).
//
// Operands: A = activation codes (rows m), B = weight codes (columns n). A
// lane holds 16 int8 of one row / column for one half of the block; the
// 4-bit weights are unpacked in registers to the same 0,2,4,6,1,3,5,7 order
// the activation codes are stored in, so A and B slots pair up element by
// element without byte permutes.
#include "qblk_device.h"

namespace qblk {
namespace {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v16i __attribute__((ext_vector_type(16)));

constexpr int BM = 128;        // activation rows per workgroup
constexpr int BN = 128;        // weight rows per workgroup
constexpr int KB = 8;          // 32-blocks per K step (one Q4_K super-block)
constexpr int kThreads = 256;  // 4 waves, 2 x 2, each 64 x 64

template <int TYPE>
struct Tile {
  static constexpr int kQuantBytes = TYPE == kQ8_0 ? 32 * KB : 16 * KB;  // per row per step
};

template <int TYPE>
__global__ __launch_bounds__(kThreads) void gemm_kernel(WeightView W, int64_t n, int64_t nb,
                                                        ActView A, int64_t m,
                                                        float* __restrict__ y, int64_t ldy) {
  constexpr int QB = Tile<TYPE>::kQuantBytes;
  __shared__ __attribute__((aligned(16))) uint8_t s_a[BM][32 * KB + 16];  // activation codes (+16: bank skew)
  __shared__ __attribute__((aligned(16))) float2 s_ads[BM][KB];       // (d, sum)
  __shared__ __attribute__((aligned(16))) uint8_t s_w[BN][QB + 16];   // weight codes (+16: bank skew)
  __shared__ __attribute__((aligned(16))) uint32_t s_wh[BN][KB];      // weight scales / header

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wm0 = (wave >> 1) * 64;  // wave's row offset in the tile
  const int wn0 = (wave & 1) * 64;   // wave's column offset in the tile
  const int64_t m0 = static_cast<int64_t>(blockIdx.y) * BM;
  const int64_t n0 = static_cast<int64_t>(blockIdx.x) * BN;
  const int half = lane >> 5;  // which 16 elements of a block this lane holds
  const int l32 = lane & 31;

  float acc[2][2][16];
#pragma unroll
  for (int a = 0; a < 2; ++a)
#pragma unroll
    for (int b = 0; b < 2; ++b)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[a][b][v] = 0.0f;

  const int64_t steps = (nb + KB - 1) / KB;
  for (int64_t st = 0; st < steps; ++st) {
    const int64_t blk0 = st * KB;
    const int nblk = static_cast<int>(nb - blk0 < KB ? nb - blk0 : KB);

    // ---- global -> LDS
    // activation codes: BM rows x (32*nblk) bytes, 16 B per thread-load
    for (int i = tid; i < BM * 2 * KB; i += kThreads) {
      const int r = i / (2 * KB);
      const int c = i % (2 * KB);  // 16-byte chunk within the step
      if (c < 2 * nblk) {
        const int64_t gm = m0 + r < m ? m0 + r : m - 1;
        *reinterpret_cast<uint4*>(&s_a[r][16 * c]) = load16(A.codes(gm, blk0) + 16 * c);
      }
    }
    for (int i = tid; i < BM * KB; i += kThreads) {
      const int r = i / KB;
      const int c = i % KB;
      if (c < nblk) {
        const int64_t gm = m0 + r < m ? m0 + r : m - 1;
        s_ads[r][c] = A.dsum(gm, blk0 + c);
      }
    }
    // weight codes
    for (int i = tid; i < BN * (QB / 16); i += kThreads) {
      const int r = i / (QB / 16);
      const int c = i % (QB / 16);
      const int per_blk = QB / 16 / KB;  // 16-byte chunks per block (1 or 2)
      if (c < per_blk * nblk) {
        const int64_t gn = n0 + r < n ? n0 + r : n - 1;
        const uint8_t* src = W.row(gn) + W.hdr_bytes + (QB / KB) * blk0 + 16 * c;
        *reinterpret_cast<uint4*>(&s_w[r][16 * c]) = load_stream16(src);
      }
    }
    // weight scales: Q4_K one 16-byte header per step, else one fp32 per block
    for (int i = tid; i < BN * KB; i += kThreads) {
      const int r = i / KB;
      const int c = i % KB;
      const int64_t gn = n0 + r < n ? n0 + r : n - 1;
      if constexpr (TYPE == kQ4_K) {
        if (c < 4) s_wh[r][c] = reinterpret_cast<const uint32_t*>(W.row(gn) + 16 * st)[c];
      } else {
        if (c < nblk) s_wh[r][c] = reinterpret_cast<const uint32_t*>(W.row(gn))[blk0 + c];
      }
    }
    __syncthreads();

    // ---- per block: MFMA on the 2 x 2 tiles, then the fp32 scale epilogue
    for (int j = 0; j < nblk; ++j) {
      v4i bop[2];
      float sw[2], wm[2];
#pragma unroll
      for (int tn = 0; tn < 2; ++tn) {
        const int r = wn0 + 32 * tn + l32;
        if constexpr (TYPE == kQ8_0) {
          const uint4 w = *reinterpret_cast<const uint4*>(&s_w[r][32 * j + 16 * half]);
          bop[tn] = v4i{static_cast<int>(w.x), static_cast<int>(w.y), static_cast<int>(w.z),
                        static_cast<int>(w.w)};
        } else {
          const uint2 w = *reinterpret_cast<const uint2*>(&s_w[r][16 * j + 8 * half]);
          const uint32_t msk = 0x0F0F0F0Fu;
          bop[tn] = v4i{static_cast<int>(w.x & msk), static_cast<int>((w.x >> 4) & msk),
                        static_cast<int>(w.y & msk), static_cast<int>((w.y >> 4) & msk)};
        }
        if constexpr (TYPE == kQ4_K) {
          const uint4 h = make_uint4(s_wh[r][0], s_wh[r][1], s_wh[r][2], s_wh[r][3]);
          sw[tn] = half_bits_to_float(h.x) * static_cast<float>(q4k_sc(h, j));
          wm[tn] = half_bits_to_float(h.x >> 16) * static_cast<float>(q4k_mn(h, j));
        } else {
          sw[tn] = __uint_as_float(s_wh[r][j]);
          wm[tn] = 0.0f;
        }
      }
#pragma unroll
      for (int tm = 0; tm < 2; ++tm) {
        const int ra = wm0 + 32 * tm + l32;
        const uint4 a = *reinterpret_cast<const uint4*>(&s_a[ra][32 * j + 16 * half]);
        const v4i aop = v4i{static_cast<int>(a.x), static_cast<int>(a.y), static_cast<int>(a.z),
                            static_cast<int>(a.w)};
#pragma unroll
        for (int tn = 0; tn < 2; ++tn) {
          v16i c = {0};
          c = __builtin_amdgcn_mfma_i32_32x32x32_i8(aop, bop[tn], c, 0, 0, 0);
#pragma unroll
          for (int v = 0; v < 16; ++v) {
            const int rm = wm0 + 32 * tm + 8 * (v >> 2) + 4 * half + (v & 3);
            const float2 ds = s_ads[rm][j];
            const int asum = __float_as_int(ds.y);
            if constexpr (TYPE == kQ4_K) {
              acc[tm][tn][v] = fmaf(ds.x, fmaf(sw[tn], static_cast<float>(c[v]),
                                               wm[tn] * static_cast<float>(asum)),
                                    acc[tm][tn][v]);
            } else if constexpr (TYPE == kQ4_0) {
              acc[tm][tn][v] = fmaf(ds.x * sw[tn], static_cast<float>(c[v] - 8 * asum),
                                    acc[tm][tn][v]);
            } else {
              acc[tm][tn][v] = fmaf(ds.x * sw[tn], static_cast<float>(c[v]), acc[tm][tn][v]);
            }
          }
        }
      }
    }
    __syncthreads();
  }

  // ---- store: lane holds column n = l32 and 16 rows of each 32 x 32 tile
#pragma unroll
  for (int tm = 0; tm < 2; ++tm)
#pragma unroll
    for (int tn = 0; tn < 2; ++tn) {
      const int64_t gn = n0 + wn0 + 32 * tn + l32;
      if (gn >= n) continue;
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int64_t gm = m0 + wm0 + 32 * tm + 8 * (v >> 2) + 4 * half + (v & 3);
        if (gm < m) y[gm * ldy + gn] = acc[tm][tn][v];
      }
    }
}

}  // namespace

hipError_t launch_gemm(int type, const void* wq, int64_t n, int64_t k, const void* xq, int64_t m,
                       float* y, int64_t ldy, hipStream_t s) {
  WeightView W;
  W.base = static_cast<const uint8_t*>(wq);
  W.row_bytes = row_bytes(type, k);
  W.hdr_bytes = header_bytes(type, k);
  const ActView A = make_act(xq, m, k);
  const int64_t nb = k / 32;
  const dim3 grid(static_cast<uint32_t>((n + BN - 1) / BN), static_cast<uint32_t>((m + BM - 1) / BM));
  switch (type) {
    case kQ4_0: hipLaunchKernelGGL(gemm_kernel<kQ4_0>, grid, dim3(kThreads), 0, s, W, n, nb, A, m, y, ldy); break;
    case kQ8_0: hipLaunchKernelGGL(gemm_kernel<kQ8_0>, grid, dim3(kThreads), 0, s, W, n, nb, A, m, y, ldy); break;
    default: hipLaunchKernelGGL(gemm_kernel<kQ4_K>, grid, dim3(kThreads), 0, s, W, n, nb, A, m, y, ldy); break;
  }
  return hipGetLastError();
}

}  // namespace qblk
