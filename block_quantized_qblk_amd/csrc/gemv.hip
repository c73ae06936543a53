// Decode-path product y[b][n] = sum_j scale * intdot(block j), few activation
// rows. HBM-bound: every packed weight byte is read exactly once.
//
// Integer dot inside each 32-block, fp32 scales outside it ("llama.cpp 推理
// 引擎", §6.4; wmrh.cn "bare engine" article, §2.2 int4 x int8 dot); Q4_K
// sub-block scale d*sc_j and min d_min*mn_j per §5.5.
//
// Mapping: one wave per weight row. Lane l takes 32-blocks l, l+64, l+128...
// so one 16-byte load per lane covers 64 consecutive blocks of 4-bit codes:
// each wave load is a contiguous KiB of the row. Per block: v_dot4_i32_i8 on
// unpacked nibbles (or int8 codes), then one or two fp32 FMAs with the block
// scales; a wave reduction at the end.
#include "qblk_device.h"

namespace qblk {
namespace {

constexpr int kWavesPerBlock = 4;

template <int TYPE, int B>
__global__ __launch_bounds__(256) void gemv_kernel(WeightView W, int64_t n, int64_t nb, ActView A,
                                                   float* __restrict__ y, int64_t ldy) {
  const int lane = threadIdx.x & 63;
  const int64_t row = static_cast<int64_t>(blockIdx.x) * kWavesPerBlock + (threadIdx.x >> 6);
  if (row >= n) return;  // whole wave
  const uint8_t* wrow = W.row(row);
  const uint8_t* wquant = wrow + W.hdr_bytes;

  float acc[B];
#pragma unroll
  for (int b = 0; b < B; ++b) acc[b] = 0.0f;

  for (int64_t blk = lane; blk < nb; blk += 64) {
    if constexpr (TYPE == kQ4_K) {
      const int j = static_cast<int>(blk & 7);
      const uint4 h = load16(wrow + 16 * (blk >> 3));
      const uint4 w = load_stream16(wquant + 16 * blk);
      const float d = half_bits_to_float(h.x);
      const float dmin = half_bits_to_float(h.x >> 16);
      const float sw = d * static_cast<float>(q4k_sc(h, j));
      const float wm = dmin * static_cast<float>(q4k_mn(h, j));
#pragma unroll
      for (int b = 0; b < B; ++b) {
        const uint8_t* ap = A.codes(b, blk);
        const uint4 a0 = load16(ap);
        const uint4 a1 = load16(ap + 16);
        const float2 ds = A.dsum(b, blk);
        const int S = dot_nib32(w, a0, a1, 0);
        const float asum = static_cast<float>(__float_as_int(ds.y));
        acc[b] = fmaf(ds.x, fmaf(sw, static_cast<float>(S), wm * asum), acc[b]);
      }
    } else if constexpr (TYPE == kQ4_0) {
      const float dw = __uint_as_float(load_stream4(wrow + 4 * blk));
      const uint4 w = load_stream16(wquant + 16 * blk);
#pragma unroll
      for (int b = 0; b < B; ++b) {
        const uint8_t* ap = A.codes(b, blk);
        const uint4 a0 = load16(ap);
        const uint4 a1 = load16(ap + 16);
        const float2 ds = A.dsum(b, blk);
        const int S = dot_nib32(w, a0, a1, 0) - 8 * __float_as_int(ds.y);
        acc[b] = fmaf(dw * ds.x, static_cast<float>(S), acc[b]);
      }
    } else {  // kQ8_0
      const float dw = __uint_as_float(load_stream4(wrow + 4 * blk));
      const uint4 w0 = load_stream16(wquant + 32 * blk);
      const uint4 w1 = load_stream16(wquant + 32 * blk + 16);
#pragma unroll
      for (int b = 0; b < B; ++b) {
        const uint8_t* ap = A.codes(b, blk);
        const uint4 a0 = load16(ap);
        const uint4 a1 = load16(ap + 16);
        const float2 ds = A.dsum(b, blk);
        const int S = dot_i8x32(w0, w1, a0, a1, 0);
        acc[b] = fmaf(dw * ds.x, static_cast<float>(S), acc[b]);
      }
    }
  }

#pragma unroll
  for (int b = 0; b < B; ++b) {
    const float s = wave_sum(acc[b]);
    if (lane == 0) y[b * ldy + row] = s;
  }
}

template <int TYPE, int B>
hipError_t launch_typed(WeightView W, int64_t n, int64_t nb, ActView A, float* y, int64_t ldy,
                        hipStream_t s) {
  const int64_t grid = (n + kWavesPerBlock - 1) / kWavesPerBlock;
  hipLaunchKernelGGL((gemv_kernel<TYPE, B>), dim3(static_cast<uint32_t>(grid)),
                     dim3(64 * kWavesPerBlock), 0, s, W, n, nb, A, y, ldy);
  return hipGetLastError();
}

template <int TYPE>
hipError_t launch_batch(int b, WeightView W, int64_t n, int64_t nb, ActView A, float* y,
                        int64_t ldy, hipStream_t s) {
  switch (b) {
    case 1: return launch_typed<TYPE, 1>(W, n, nb, A, y, ldy, s);
    case 2: return launch_typed<TYPE, 2>(W, n, nb, A, y, ldy, s);
    case 3: return launch_typed<TYPE, 3>(W, n, nb, A, y, ldy, s);
    case 4: return launch_typed<TYPE, 4>(W, n, nb, A, y, ldy, s);
    case 5: return launch_typed<TYPE, 5>(W, n, nb, A, y, ldy, s);
    case 6: return launch_typed<TYPE, 6>(W, n, nb, A, y, ldy, s);
    case 7: return launch_typed<TYPE, 7>(W, n, nb, A, y, ldy, s);
    default: return launch_typed<TYPE, 8>(W, n, nb, A, y, ldy, s);
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
