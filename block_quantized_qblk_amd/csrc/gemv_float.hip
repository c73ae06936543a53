// Decode product with fp32 activations, no activation quantization:
// y[b][n] = sum_k dequant(W)[n][k] * x[b][k].
//
// This is the form of the pages' scalar Q4_0 dot ("llama.cpp 推理引擎",
// §6.4): each weight is decoded in place (nibble - 8, times the block scale)
// and multiplied by a float activation; for Q4_K the sub-block scale and min
// of §5.5 apply (w = d*sc_j*q + d_min*mn_j). The weights stay packed in HBM;
// per block the lane converts its codes to fp32 and accumulates
//   d * (sum_i q_i x_i - 8 sum_i x_i)        (Q4_0, Q4_0_F16)
//   d * sum_i q_i x_i                         (Q8_0)
//   d*sc_j * sum_i q_i x_i + d_min*mn_j * sum_i x_i   (Q4_K)
// so every block costs one conversion and one FMA per element plus its block
// sum of x.
//
// Mapping as in the quantized GEMV: a wave owns R weight rows and walks them
// in chunks of 64 blocks, lane l taking block c + l with one 16-byte
// (nibbles) or two (Q8_0) nontemporal loads per row; the lane's 32 activations
// of that block are read once per batch row (8 float4 loads) and shared by the
// R rows. When they fit in 64 KiB the workgroup first copies the activation
// rows into LDS, so its four waves read them from there rather than each from
// L2 (Q8_0 14336 x 4096: 17.4 against 22.4 us). A DPP wave reduction ends each
// (row, batch) sum.
#include "qblk_device.h"

namespace qblk {
namespace {

constexpr int kWaves = 4;

// Block data of one weight row for one lane.
template <int TYPE>
struct FBlock {
  uint4 q0;       // codes (16 bytes; Q8_0: first 16)
  uint4 q1;       // Q8_0: last 16 bytes
  float d;        // block scale (Q4_K: d * sc_j)
  float dm;       // Q4_K: d_min * mn_j; Q4_0: -8 d
};

template <int TYPE>
__device__ __forceinline__ FBlock<TYPE> load_fblock(const uint8_t* row, int64_t hdr, int64_t blk) {
  FBlock<TYPE> f;
  f.q1 = make_uint4(0, 0, 0, 0);
  f.dm = 0.0f;
  if constexpr (TYPE == kQ8_0) {
    const uint8_t* p = row + hdr + 32 * blk;
    f.q0 = load_stream16(p);
    f.q1 = load_stream16(p + 16);
    f.d = __uint_as_float(load_stream4(row + 4 * blk));
  } else if constexpr (TYPE == kQ4_K) {
    f.q0 = load_stream16(row + hdr + 16 * blk);
    const uint4 h = load16(row + 16 * (blk >> 3));
    const int j = static_cast<int>(blk & 7);
    f.d = half_bits_to_float(h.x) * static_cast<float>(q4k_sc(h, j));
    f.dm = half_bits_to_float(h.x >> 16) * static_cast<float>(q4k_mn(h, j));
  } else {
    f.q0 = load_stream16(row + hdr + 16 * blk);
    f.d = TYPE == kQ4_0H ? half_bits_to_float(load_stream2(row + 2 * blk))
                         : __uint_as_float(load_stream4(row + 4 * blk));
    f.dm = -8.0f * f.d;  // codes are nibble - 8
  }
  return f;
}

// byte i of w as fp32 (one v_cvt_f32_ubyte<i>)
__device__ __forceinline__ float ubyte(uint32_t w, int i) { return static_cast<float>((w >> (8 * i)) & 0xFFu); }

// sum over the 8 elements 8g..8g+7 held as (low part = elements 8g + 2i,
// high part = elements 8g + 2i + 1, i = 0..3) of a code dword pair.
__device__ __forceinline__ float dot8_unsigned(uint32_t lo, uint32_t hi, const float4& xa, const float4& xb,
                                               float acc) {
  // lo byte i is element 2i, hi byte i is element 2i + 1 of the group
  acc = fmaf(ubyte(lo, 0), xa.x, acc);
  acc = fmaf(ubyte(hi, 0), xa.y, acc);
  acc = fmaf(ubyte(lo, 1), xa.z, acc);
  acc = fmaf(ubyte(hi, 1), xa.w, acc);
  acc = fmaf(ubyte(lo, 2), xb.x, acc);
  acc = fmaf(ubyte(hi, 2), xb.y, acc);
  acc = fmaf(ubyte(lo, 3), xb.z, acc);
  acc = fmaf(ubyte(hi, 3), xb.w, acc);
  return acc;
}

__device__ __forceinline__ float sbyte(uint32_t w, int i) {
  return static_cast<float>(static_cast<int8_t>(static_cast<uint8_t>(w >> (8 * i))));
}

__device__ __forceinline__ float dot8_signed(uint32_t lo, uint32_t hi, const float4& xa, const float4& xb,
                                             float acc) {
  acc = fmaf(sbyte(lo, 0), xa.x, acc);
  acc = fmaf(sbyte(hi, 0), xa.y, acc);
  acc = fmaf(sbyte(lo, 1), xa.z, acc);
  acc = fmaf(sbyte(hi, 1), xa.w, acc);
  acc = fmaf(sbyte(lo, 2), xb.x, acc);
  acc = fmaf(sbyte(hi, 2), xb.y, acc);
  acc = fmaf(sbyte(lo, 3), xb.z, acc);
  acc = fmaf(sbyte(hi, 3), xb.w, acc);
  return acc;
}

// sum_i q_i x_i over one block; x holds the block's 32 activations in order.
template <int TYPE>
__device__ __forceinline__ float block_dot(const FBlock<TYPE>& f, const float4 (&x)[8]) {
  float s = 0.0f;
  if constexpr (TYPE == kQ8_0) {
    // groups of 8 stored as elements 0,2,4,6 then 1,3,5,7
    s = dot8_signed(f.q0.x, f.q0.y, x[0], x[1], s);
    s = dot8_signed(f.q0.z, f.q0.w, x[2], x[3], s);
    s = dot8_signed(f.q1.x, f.q1.y, x[4], x[5], s);
    s = dot8_signed(f.q1.z, f.q1.w, x[6], x[7], s);
  } else {
    // byte t = element 2t (low nibble) | element 2t + 1 (high nibble)
    const uint32_t m = 0x0F0F0F0Fu;
    s = dot8_unsigned(f.q0.x & m, (f.q0.x >> 4) & m, x[0], x[1], s);
    s = dot8_unsigned(f.q0.y & m, (f.q0.y >> 4) & m, x[2], x[3], s);
    s = dot8_unsigned(f.q0.z & m, (f.q0.z >> 4) & m, x[4], x[5], s);
    s = dot8_unsigned(f.q0.w & m, (f.q0.w >> 4) & m, x[6], x[7], s);
  }
  return s;
}

// LDS bytes of the staged activation rows: B rows of nb blocks, each block's
// 32 floats as 8 float4 units laid out unit-major per 64-block chunk, so
// that a wave's read of unit i of 64 consecutive blocks is one contiguous
// KiB (lane l at +16 l, free of bank conflicts).
__host__ __device__ inline uint32_t xlds_bytes(int b, int64_t nb) {
  return static_cast<uint32_t>(b * ((nb + 63) / 64) * 64 * 128);
}
constexpr uint32_t kXLdsMax = 65536;  // 4 rows of K = 4096 (Q4_K 14336 x 4096 at batch 4: 24.6 against 36.2 us)

template <int TYPE, int R, int B, bool XLDS>
__global__ __launch_bounds__(64 * kWaves) void gemv_float_kernel(WeightView W, int64_t n, int64_t nb,
                                                                  const float* __restrict__ x, int64_t ldx,
                                                                  int batch, float* __restrict__ y,
                                                                  int64_t ldy) {
  extern __shared__ __attribute__((aligned(16))) float4 xs[];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int64_t row0 = (static_cast<int64_t>(blockIdx.x) * kWaves + wave) * R;
  const int64_t nc = (nb + 63) / 64;  // 64-block chunks per row
  if constexpr (XLDS) {
    // the workgroup copies the activation rows into LDS once: float4 unit u
    // of block blk of row b goes to ((b * nc + blk / 64) * 8 + u) * 64 + blk % 64
    for (int b = 0; b < B; ++b) {
      const int bb = b < batch ? b : batch - 1;
      const float4* xp = reinterpret_cast<const float4*>(x + bb * ldx);
      for (int64_t q = threadIdx.x; q < nb * 8; q += 64 * kWaves) {
        const int64_t blk = q >> 3;
        const int u = static_cast<int>(q & 7);
        xs[((b * nc + (blk >> 6)) * 8 + u) * 64 + (blk & 63)] = xp[q];
      }
    }
    __syncthreads();
  }
  if (row0 >= n) return;  // wave-uniform; no workgroup barrier follows

  float acc[R][B];
#pragma unroll
  for (int r = 0; r < R; ++r)
#pragma unroll
    for (int b = 0; b < B; ++b) acc[r][b] = 0.0f;

  for (int64_t c = 0; c < nb; c += 64) {
    const int64_t blk = c + lane;
    if (blk < nb) {
      FBlock<TYPE> f[R];
#pragma unroll
      for (int r = 0; r < R; ++r) {
        const int64_t row = row0 + r < n ? row0 + r : n - 1;  // a clamped row is not stored
        f[r] = load_fblock<TYPE>(W.row(row), W.hdr_bytes, blk);
      }
#pragma unroll
      for (int b = 0; b < B; ++b) {
        const int bb = b < batch ? b : batch - 1;  // padded batch rows are not stored
        float4 xv[8];
        if constexpr (XLDS) {
          const float4* xl = xs + (b * nc + (c >> 6)) * 512 + lane;
#pragma unroll
          for (int i = 0; i < 8; ++i) xv[i] = xl[64 * i];
        } else {
          const float4* xp = reinterpret_cast<const float4*>(x + bb * ldx + 32 * blk);
#pragma unroll
          for (int i = 0; i < 8; ++i) xv[i] = xp[i];
        }
        float sx = 0.0f;
        if constexpr (TYPE != kQ8_0) {
#pragma unroll
          for (int i = 0; i < 8; ++i) sx += (xv[i].x + xv[i].y) + (xv[i].z + xv[i].w);
        }
#pragma unroll
        for (int r = 0; r < R; ++r) {
          const float dq = block_dot<TYPE>(f[r], xv);
          float t = f[r].d * dq;
          if constexpr (TYPE != kQ8_0) t = fmaf(f[r].dm, sx, t);
          acc[r][b] += t;
        }
      }
    }
  }

#pragma unroll
  for (int r = 0; r < R; ++r)
#pragma unroll
    for (int b = 0; b < B; ++b) {
      const float s = wave_sum_dpp(acc[r][b]);  // lands in lane 63
      if (lane == 63 && row0 + r < n && b < batch) y[b * ldy + row0 + r] = s;
    }
}

template <int TYPE, int R, int B>
void launch_rb(const WeightView& W, int64_t n, int64_t nb, const float* x, int64_t ldx, int batch, float* y,
               int64_t ldy, hipStream_t s) {
  const int64_t rows_per_wg = static_cast<int64_t>(kWaves) * R;
  const dim3 grid(static_cast<uint32_t>((n + rows_per_wg - 1) / rows_per_wg));
  const uint32_t lds = xlds_bytes(B, nb);
  if (lds <= kXLdsMax)
    hipLaunchKernelGGL((gemv_float_kernel<TYPE, R, B, true>), grid, dim3(64 * kWaves), lds, s, W, n, nb, x,
                       ldx, batch, y, ldy);
  else
    hipLaunchKernelGGL((gemv_float_kernel<TYPE, R, B, false>), grid, dim3(64 * kWaves), 0, s, W, n, nb, x,
                       ldx, batch, y, ldy);
}

template <int TYPE>
void launch_t(const WeightView& W, int64_t n, int64_t nb, const float* x, int64_t ldx, int batch, float* y,
              int64_t ldy, hipStream_t s) {
  // 4 rows per wave share each activation read (measured on MI355X: 1.2-1.5x
  // faster than 2 at batch 1 and 4; 8 is no better)
  if (batch == 1) launch_rb<TYPE, 4, 1>(W, n, nb, x, ldx, batch, y, ldy, s);
  else if (batch == 2) launch_rb<TYPE, 4, 2>(W, n, nb, x, ldx, batch, y, ldy, s);
  else if (batch <= 4) launch_rb<TYPE, 4, 4>(W, n, nb, x, ldx, batch, y, ldy, s);
  else launch_rb<TYPE, 2, 8>(W, n, nb, x, ldx, batch, y, ldy, s);
}

}  // namespace

hipError_t launch_gemv_float(int type, const void* wq, int64_t n, int64_t k, const float* x, int64_t ldx,
                             int64_t batch, float* y, int64_t ldy, hipStream_t s) {
  WeightView W;
  W.base = static_cast<const uint8_t*>(wq);
  W.row_bytes = row_bytes(type, k);
  W.hdr_bytes = header_bytes(type, k);
  const int64_t nb = k / 32;
  // one launch per 8 activation rows
  for (int64_t b0 = 0; b0 < batch; b0 += 8) {
    const int b = static_cast<int>(batch - b0 < 8 ? batch - b0 : 8);
    const float* xb = x + b0 * ldx;
    float* yb = y + b0 * ldy;
    switch (type) {
      case kQ4_0: launch_t<kQ4_0>(W, n, nb, xb, ldx, b, yb, ldy, s); break;
      case kQ8_0: launch_t<kQ8_0>(W, n, nb, xb, ldx, b, yb, ldy, s); break;
      case kQ4_0H: launch_t<kQ4_0H>(W, n, nb, xb, ldx, b, yb, ldy, s); break;
      default: launch_t<kQ4_K>(W, n, nb, xb, ldx, b, yb, ldy, s); break;
    }
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace qblk
