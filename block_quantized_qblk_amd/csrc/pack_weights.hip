// Weight quantization and packing (setup step, not on the per-token path).
//
// Q4_0 / Q8_0: "llama.cpp 推理引擎" §5.1 (symmetric rule) with b = 4 (codes in
// [-7, 7], stored as nibble q + 8, §5.3 and the §6.4 nibble order) or b = 8
// (§5.4), fp32 scale, decisions in fp32 with IEEE division. Q4_0_F16 (§5.3's
// own block): the same with the scale rounded to the nearest fp16 (ties to
// even, saturating at 65504) before the codes are taken against it.
//
// Q4_K: §5.2 (asymmetric rule, zero point = block minimum) inside the §5.5
// hierarchy: 256-element super-blocks of 8 sub-blocks of 32 (also "llama.cpp：
// 一个人、一个周末…", section 量化是怎么做到的？), 6-bit sub-block scale and min
// codes under fp16 super-block scales. Every decision is taken in fp64 with
// exact or correctly rounded operations, so the packed bytes are a pure
// function of the fp32 input:
//   m_j = max(0, -min_j)                       zero point -m_j, never above 0
//   h   = smallest fp16 with 63*h >= max_j m_j  (stored as d_min = -h)
//   mn_j = smallest code with mn_j*h >= m_j,   M_j = mn_j*h
//   t_j = max_j + M_j                          range the 16 levels must span
//   d   = smallest fp16 with 945*d >= max_j t_j
//   sc_j = smallest code with 15*sc_j*d >= t_j, S_j = sc_j*d
//   q = clamp(round((x + M_j) / S_j), 0, 15)   (0 when S_j == 0)
// so |x - ((d*sc_j)*q + d_min*mn_j)| <= S_j / 2 for every element.
#include "qblk_device.h"

#pragma clang fp contract(off)

namespace qblk {
namespace {

__device__ __forceinline__ uint2 pack_group8(const int (&q)[8]) {
  uint2 r;
  r.x = (q[0] & 255u) | (q[2] & 255u) << 8 | (q[4] & 255u) << 16 | (q[6] & 255u) << 24;
  r.y = (q[1] & 255u) | (q[3] & 255u) << 8 | (q[5] & 255u) << 16 | (q[7] & 255u) << 24;
  return r;
}

// Q4_0 (QMAX 7) and Q8_0 (QMAX 127), F16: Q4_0_F16; four lanes per 32-block.
template <int QMAX, bool F16 = false>
__global__ __launch_bounds__(256) void pack_sym_kernel(const float* __restrict__ w, int64_t n,
                                                       int64_t k, int64_t ldw,
                                                       uint8_t* __restrict__ wq, int64_t ob,
                                                       int64_t hb) {
  const int64_t nb = k / 32;
  const int64_t gid = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  const int64_t blk_all = gid >> 2;
  if (blk_all >= n * nb) return;
  const int sub = static_cast<int>(gid & 3);
  const int64_t row = blk_all / nb;
  const int64_t blk = blk_all - row * nb;

  const float* src = w + row * ldw + 32 * blk + 8 * sub;
  const float4 v0 = *reinterpret_cast<const float4*>(src);
  const float4 v1 = *reinterpret_cast<const float4*>(src + 4);
  const float e[8] = {v0.x, v0.y, v0.z, v0.w, v1.x, v1.y, v1.z, v1.w};

  float amax = 0.0f;
#pragma unroll
  for (int i = 0; i < 8; ++i) amax = fmaxf(amax, fabsf(e[i]));
  amax = fmaxf(amax, __shfl_xor(amax, 1, 64));
  amax = fmaxf(amax, __shfl_xor(amax, 2, 64));
  float d = __fdiv_rn(amax, static_cast<float>(QMAX));
  _Float16 d16 = 0;
  if constexpr (F16) {
    d16 = static_cast<_Float16>(fminf(d, 65504.0f));  // round to nearest even
    if (d > 65504.0f) d16 = static_cast<_Float16>(65504.0f);
    d = static_cast<float>(d16);
  }

  int q[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    int qi = 0;
    if (d != 0.0f) {
      float r = roundf(__fdiv_rn(e[i], d));
      r = fminf(fmaxf(r, -static_cast<float>(QMAX)), static_cast<float>(QMAX));
      qi = static_cast<int>(r);
    }
    q[i] = qi;
  }

  uint8_t* dst = wq + row * ob;  // ob: bytes between output rows
  if constexpr (F16) {
    if (sub == 0) *reinterpret_cast<_Float16*>(dst + 2 * blk) = d16;
    // zero the padding at the end of the header region (up to 7 halves)
    if (blk == nb - 1) {
      if (2 * (nb + sub) < hb) *reinterpret_cast<uint16_t*>(dst + 2 * (nb + sub)) = 0;
      if (2 * (nb + sub + 4) < hb) *reinterpret_cast<uint16_t*>(dst + 2 * (nb + sub + 4)) = 0;
    }
  } else {
    if (sub == 0) *reinterpret_cast<float*>(dst + 4 * blk) = d;
    // zero the padding at the end of the header region
    if (blk == nb - 1 && sub > 0 && 4 * (nb + sub - 1) < hb)
      *reinterpret_cast<uint32_t*>(dst + 4 * (nb + sub - 1)) = 0u;
  }

  if constexpr (QMAX == 7) {
    uint32_t packed = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i)
      packed |= ((static_cast<uint32_t>(q[2 * i] + 8)) | (static_cast<uint32_t>(q[2 * i + 1] + 8) << 4))
                << (8 * i);
    *reinterpret_cast<uint32_t*>(dst + hb + 16 * blk + 4 * sub) = packed;
  } else {
    *reinterpret_cast<uint2*>(dst + hb + 32 * blk + 8 * sub) = pack_group8(q);
  }
}

// ---------------------------------------------------------------- Q4_K

// Value of an IEEE binary16 bit pattern (finite), exactly, in fp64.
__device__ __forceinline__ double f16_value(int b) {
  const int e = (b >> 10) & 31;
  const int mnt = b & 1023;
  const double v = e == 0 ? static_cast<double>(mnt) * 0x1p-24
                          : ldexp(static_cast<double>(1024 + mnt), e - 25);
  return (b & 0x8000) ? -v : v;
}

// Smallest non-negative fp16 h (bit pattern) with c*h >= v; saturates at the
// largest finite fp16. c*h is exact in fp64.
__device__ __forceinline__ int f16_ceil_div(double v, double c) {
  int lo = 0, hi = 0x7BFF;
  for (int it = 0; it < 16; ++it) {
    const int mid = (lo + hi) >> 1;
    if (c * f16_value(mid) >= v) {
      hi = mid;
    } else {
      lo = mid + 1;
    }
    lo = lo < hi ? lo : hi;
  }
  return hi;
}

__device__ __forceinline__ double round_half_away(double v) {
  const double a = fabs(v);
  double r = floor(a);
  if (a - r >= 0.5) r += 1.0;
  return copysign(r, v);
}

__device__ __forceinline__ double group8_max(double v, int lane) {
  (void)lane;
  v = fmax(v, __shfl_xor(v, 1, 64));
  v = fmax(v, __shfl_xor(v, 2, 64));
  v = fmax(v, __shfl_xor(v, 4, 64));
  return v;
}

// Eight lanes per super-block, lane j owns sub-block j (32 elements).
__global__ __launch_bounds__(256) void pack_q4k_kernel(const float* __restrict__ w, int64_t n,
                                                       int64_t k, int64_t ldw,
                                                       uint8_t* __restrict__ wq, int64_t ob,
                                                       int64_t hb) {
  const int64_t nsb = k / 256;
  const int64_t gid = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  const int64_t sb_all = gid >> 3;
  if (sb_all >= n * nsb) return;  // a whole 8-lane group leaves together
  const int j = static_cast<int>(gid & 7);
  const int lane = threadIdx.x & 63;
  const int64_t row = sb_all / nsb;
  const int64_t sb = sb_all - row * nsb;

  const float* src = w + row * ldw + 256 * sb + 32 * j;
  float x[32];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const float4 v = reinterpret_cast<const float4*>(src)[i];
    x[4 * i + 0] = v.x;
    x[4 * i + 1] = v.y;
    x[4 * i + 2] = v.z;
    x[4 * i + 3] = v.w;
  }
  float hi_f = x[0], lo_f = x[0];
#pragma unroll
  for (int i = 1; i < 32; ++i) {
    hi_f = fmaxf(hi_f, x[i]);
    lo_f = fminf(lo_f, x[i]);
  }
  const double hi = hi_f;
  const double m = fmax(0.0, -static_cast<double>(lo_f));

  const int dm_bits = f16_ceil_div(group8_max(m, lane), 63.0);
  const double dm = f16_value(dm_bits);
  int mn = 0;
  for (int c = 0; c < 64; ++c) mn += (static_cast<double>(c) * dm < m) ? 1 : 0;
  mn = mn < 63 ? mn : 63;
  const double M = static_cast<double>(mn) * dm;
  const double t = hi + M;

  const int d_bits = f16_ceil_div(group8_max(t, lane), 945.0);
  const double d = f16_value(d_bits);
  int sc = 0;
  for (int c = 0; c < 64; ++c) sc += (15.0 * static_cast<double>(c) * d < t) ? 1 : 0;
  sc = sc < 63 ? sc : 63;
  const double S = static_cast<double>(sc) * d;

  uint32_t nib[4] = {0u, 0u, 0u, 0u};
#pragma unroll
  for (int i = 0; i < 32; ++i) {
    int q = 0;
    if (S != 0.0) {
      double r = round_half_away((static_cast<double>(x[i]) + M) / S);
      r = fmin(fmax(r, 0.0), 15.0);
      q = static_cast<int>(r);
    }
    // byte t = i/2 of the sub-block: element 2t low nibble, 2t+1 high nibble
    nib[i >> 3] |= static_cast<uint32_t>(q) << (4 * (i & 7));
  }
  uint8_t* dst = wq + row * ob;  // ob: bytes between output rows
  *reinterpret_cast<uint4*>(dst + hb + 128 * sb + 16 * j) = make_uint4(nib[0], nib[1], nib[2], nib[3]);

  // assemble the 96-bit sc/mn field in lane j == 0 of the group
  const int base = lane & ~7;
  uint64_t f_lo = 0, f_hi = 0;
#pragma unroll
  for (int jj = 0; jj < 8; ++jj) {
    const uint64_t s_j = static_cast<uint64_t>(__shfl(sc, base + jj, 64));
    const uint64_t m_j = static_cast<uint64_t>(__shfl(mn, base + jj, 64));
    f_lo |= s_j << (6 * jj);  // bits 0..47
    const int p = 48 + 6 * jj;
    if (p + 6 <= 64) {
      f_lo |= m_j << p;
    } else if (p >= 64) {
      f_hi |= m_j << (p - 64);
    } else {
      f_lo |= m_j << p;
      f_hi |= m_j >> (64 - p);
    }
  }
  if (j == 0) {
    const uint32_t dmin_bits = dm_bits == 0 ? 0u : (static_cast<uint32_t>(dm_bits) | 0x8000u);
    uint4 h;
    h.x = static_cast<uint32_t>(d_bits) | (dmin_bits << 16);
    h.y = static_cast<uint32_t>(f_lo);
    h.z = static_cast<uint32_t>(f_lo >> 32);
    h.w = static_cast<uint32_t>(f_hi);
    *reinterpret_cast<uint4*>(dst + 16 * sb) = h;
  }
}

}  // namespace

hipError_t launch_pack_weights(int type, const float* w, int64_t n, int64_t k, int64_t ldw,
                               void* wq, int64_t out_stride, hipStream_t s) {
  const int64_t rb = out_stride;
  const int64_t hb = header_bytes(type, k);
  uint8_t* out = static_cast<uint8_t*>(wq);
  if (type == kQ4_K) {
    const int64_t threads = 8 * n * (k / 256);
    const int64_t grid = (threads + 255) / 256;
    hipLaunchKernelGGL(pack_q4k_kernel, dim3(static_cast<uint32_t>(grid)), dim3(256), 0, s, w, n,
                       k, ldw, out, rb, hb);
  } else {
    const int64_t threads = 4 * n * (k / 32);
    const int64_t grid = (threads + 255) / 256;
    if (type == kQ4_0) {
      hipLaunchKernelGGL(pack_sym_kernel<7>, dim3(static_cast<uint32_t>(grid)), dim3(256), 0, s,
                         w, n, k, ldw, out, rb, hb);
    } else if (type == kQ4_0H) {
      hipLaunchKernelGGL((pack_sym_kernel<7, true>), dim3(static_cast<uint32_t>(grid)), dim3(256),
                         0, s, w, n, k, ldw, out, rb, hb);
    } else {
      hipLaunchKernelGGL(pack_sym_kernel<127>, dim3(static_cast<uint32_t>(grid)), dim3(256), 0,
                         s, w, n, k, ldw, out, rb, hb);
    }
  }
  return hipGetLastError();
}

}  // namespace qblk
