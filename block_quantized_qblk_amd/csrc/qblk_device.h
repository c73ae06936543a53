// Device-side building blocks shared by the GEMV, GEMM and block-sum
// kernels: packed-row addressing, nibble unpack, int8 block dots and wave
// reductions. gfx950 (CDNA4, wave64) only.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "qblk_internal.h"

namespace qblk {

// ---------------------------------------------------------------- loads
// Weights are streamed exactly once per product: load them non-temporally so
// they do not evict the activations that every wave re-reads.
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ uint4 load_stream16(const uint8_t* p) {
  const u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
  return make_uint4(v.x, v.y, v.z, v.w);
}
__device__ __forceinline__ uint32_t load_stream4(const uint8_t* p) {
  return __builtin_nontemporal_load(reinterpret_cast<const uint32_t*>(p));
}
__device__ __forceinline__ uint32_t load_stream2(const uint8_t* p) {
  return __builtin_nontemporal_load(reinterpret_cast<const uint16_t*>(p));
}
__device__ __forceinline__ uint4 load16(const uint8_t* p) {
  return *reinterpret_cast<const uint4*>(p);
}

// ---------------------------------------------------------------- fp16
__device__ __forceinline__ float half_bits_to_float(uint32_t h) {
  _Float16 v = __builtin_bit_cast(_Float16, static_cast<uint16_t>(h & 0xFFFFu));
  return static_cast<float>(v);  // exact conversion
}

// ---------------------------------------------------------------- int8 dots
__device__ __forceinline__ int dot4(uint32_t a, uint32_t b, int acc) {
  return __builtin_amdgcn_sdot4(static_cast<int>(a), static_cast<int>(b), acc, false);
}

// The first product of a chain. The compiler selects the two-operand dot
// (v_dot4c_i32_i8, whose accumulator is also its destination) and so clears
// a register for every chain; the three-operand form takes the zero as an
// inline constant (one VALU instruction less per block and row: the 70B layer
// at batch 4 went from 131.9 to 130.1 us).
__device__ __forceinline__ int dot4_zero(uint32_t a, uint32_t b) {
  int r;
  asm("v_dot4_i32_i8 %0, %1, %2, 0" : "=v"(r) : "v"(a), "v"(b));
  return r;
}

// 32 4-bit codes (16 bytes, byte t = element 2t | element 2t+1 << 4) against
// 32 int8 activation codes stored in the order 0,2,4,6,1,3,5,7 per group of
// 8: the low nibbles of four bytes are elements 0,2,4,6 of the group, the
// high nibbles elements 1,3,5,7, so each dword dot needs no permute.
// Nibbles are taken as unsigned 0..15 (non-negative int8).
__device__ __forceinline__ int dot_nib32(uint4 w, uint4 a0, uint4 a1) {
  const uint32_t m = 0x0F0F0F0Fu;
  int acc = dot4_zero(w.x & m, a0.x);
  acc = dot4((w.x >> 4) & m, a0.y, acc);
  acc = dot4(w.y & m, a0.z, acc);
  acc = dot4((w.y >> 4) & m, a0.w, acc);
  acc = dot4(w.z & m, a1.x, acc);
  acc = dot4((w.z >> 4) & m, a1.y, acc);
  acc = dot4(w.w & m, a1.z, acc);
  acc = dot4((w.w >> 4) & m, a1.w, acc);
  return acc;
}

// The fp32 number 1.5 * 2^23 and its bit pattern. An int32 dot chain that
// starts from the bit pattern (instead of 0) ends at the bit pattern of the
// float 1.5 * 2^23 + S, exactly, for |S| < 2^22 (every block dot here).
constexpr int kMagicBits = 0x4B400000;
constexpr float kMagic = 12582912.0f;

// First product of a chain that starts at kMagicBits (held in a scalar
// register, the three-operand dot).
__device__ __forceinline__ int dot4_magic(uint32_t a, uint32_t b) {
  int r;
  asm("v_dot4_i32_i8 %0, %1, %2, %3" : "=v"(r) : "v"(a), "v"(b), "s"(kMagicBits));
  return r;
}

// dot_nib32 read as fp32: 1.5 * 2^23 + S, exactly.
__device__ __forceinline__ float dot_nib32_magic(uint4 w, uint4 a0, uint4 a1) {
  const uint32_t m = 0x0F0F0F0Fu;
  int acc = dot4_magic(w.x & m, a0.x);
  acc = dot4((w.x >> 4) & m, a0.y, acc);
  acc = dot4(w.y & m, a0.z, acc);
  acc = dot4((w.y >> 4) & m, a0.w, acc);
  acc = dot4(w.z & m, a1.x, acc);
  acc = dot4((w.z >> 4) & m, a1.y, acc);
  acc = dot4(w.w & m, a1.z, acc);
  acc = dot4((w.w >> 4) & m, a1.w, acc);
  return __int_as_float(acc);
}

// 32 int8 codes against 32 int8 codes, both in the same per-group order.
__device__ __forceinline__ int dot_i8x32(uint4 w0, uint4 w1, uint4 a0, uint4 a1) {
  int acc = dot4_zero(w0.x, a0.x);
  acc = dot4(w0.y, a0.y, acc);
  acc = dot4(w0.z, a0.z, acc);
  acc = dot4(w0.w, a0.w, acc);
  acc = dot4(w1.x, a1.x, acc);
  acc = dot4(w1.y, a1.y, acc);
  acc = dot4(w1.z, a1.z, acc);
  acc = dot4(w1.w, a1.w, acc);
  return acc;
}

// Q4_K header of one super-block: fp16 d, fp16 d_min, then sc_j at bits
// [6j, 6j+6) and mn_j at bits [48+6j, 48+6j+6) of the 96-bit field held in
// h.y (bits 0..31), h.z (32..63), h.w (64..95).
__device__ __forceinline__ uint32_t q4k_sc(uint4 h, int j) {
  const uint64_t lo = (static_cast<uint64_t>(h.z) << 32) | h.y;
  return static_cast<uint32_t>(lo >> (6 * j)) & 63u;
}
__device__ __forceinline__ uint32_t q4k_mn(uint4 h, int j) {
  const uint64_t hi = (static_cast<uint64_t>(h.w) << 32) | h.z;
  return static_cast<uint32_t>(hi >> (16 + 6 * j)) & 63u;
}

// ---------------------------------------------------------------- reductions
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off, 64);
  return v;
}

// DPP move of v; lanes of rows disabled by ROW_MASK read 0.
template <int CTRL, int ROW_MASK>
__device__ __forceinline__ float dpp_move(float v) {
  return __builtin_bit_cast(
      float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL, ROW_MASK, 0xF, false));
}

// Sum over the 64 lanes with DPP only; the total lands in lane 63.
//   quad_perm(1,0,3,2), quad_perm(2,3,0,1): sums of 4 lanes
//   row_half_mirror, row_mirror: sums of 8, then 16 lanes (one row)
//   row_bcast:15 into rows 1 and 3, row_bcast:31 into rows 2 and 3
__device__ __forceinline__ float wave_sum_dpp(float v) {
  v += dpp_move<0xB1, 0xF>(v);
  v += dpp_move<0x4E, 0xF>(v);
  v += dpp_move<0x141, 0xF>(v);
  v += dpp_move<0x140, 0xF>(v);
  v += dpp_move<0x142, 0xA>(v);
  v += dpp_move<0x143, 0xC>(v);
  return v;
}

// ---------------------------------------------------------------- Q8 activation quantizer
// One 32-block is quantized by four consecutive lanes, 8 elements each
// ("llama.cpp 推理引擎", §5.1 at b = 8): d = max|x| / 127 and q = round(x / d),
// both IEEE fp32 divisions (correctly rounded), round half away from zero,
// d == 0 gives q == 0. Returns the lane's 8 codes packed in the element order
// 0,2,4,6 | 1,3,5,7; the block's scale and code sum come back in d / sum
// (valid in every lane of the group). The group is an aligned quad of lanes
// (lanes 4i..4i+3) and all four must be active.
struct Q8Group {
  uint2 codes;
  float d;
  int sum;
};

// Value of lane (l ^ 1) / (l ^ 2) within each aligned quad of lanes (DPP
// quad_perm), for the 4-lane groups of the quantizer.
template <int CTRL>
__device__ __forceinline__ int quad_swap(int v) {
  return __builtin_amdgcn_mov_dpp(v, CTRL, 0xF, 0xF, true);
}
template <int CTRL>
__device__ __forceinline__ float quad_swap(float v) {
  return __builtin_bit_cast(float, quad_swap<CTRL>(__builtin_bit_cast(int, v)));
}
constexpr int kQuadXor1 = 0xB1;  // quad_perm [1,0,3,2]
constexpr int kQuadXor2 = 0x4E;  // quad_perm [2,3,0,1]

__device__ __forceinline__ Q8Group quantize_group8(const float (&e)[8]) {
#pragma clang fp contract(off)
  float amax = 0.0f;
#pragma unroll
  for (int i = 0; i < 8; ++i) amax = fmaxf(amax, fabsf(e[i]));
  amax = fmaxf(amax, quad_swap<kQuadXor1>(amax));
  amax = fmaxf(amax, quad_swap<kQuadXor2>(amax));
  Q8Group r;
  r.d = __fdiv_rn(amax, 127.0f);
  int q[8];
  int s = 0;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    int qi = 0;
    if (r.d != 0.0f) {
      float t = roundf(__fdiv_rn(e[i], r.d));  // half away from zero
      t = fminf(fmaxf(t, -127.0f), 127.0f);
      qi = static_cast<int>(t);
    }
    q[i] = qi;
    s += qi;
  }
  s += quad_swap<kQuadXor1>(s);
  s += quad_swap<kQuadXor2>(s);
  r.sum = s;
  r.codes.x = (q[0] & 255u) | (q[2] & 255u) << 8 | (q[4] & 255u) << 16 | (q[6] & 255u) << 24;
  r.codes.y = (q[1] & 255u) | (q[3] & 255u) << 8 | (q[5] & 255u) << 16 | (q[7] & 255u) << 24;
  return r;
}

// Activation buffer views (m rows of k): codes, then (d, sum) pairs.
struct ActView {
  const uint8_t* q;   // [m][k] int8 codes
  const uint8_t* ds;  // [m][nb] (fp32 d, int32 sum)
  int64_t k;
  int64_t nb;
  __device__ __forceinline__ const uint8_t* codes(int64_t row, int64_t blk) const {
    return q + row * k + 32 * blk;
  }
  __device__ __forceinline__ float2 dsum(int64_t row, int64_t blk) const {
    return *reinterpret_cast<const float2*>(ds + 8 * (row * nb + blk));
  }
};

__host__ __device__ inline ActView make_act(const void* xq, int64_t m, int64_t k) {
  ActView a;
  a.q = static_cast<const uint8_t*>(xq);
  a.ds = a.q + m * k;
  a.k = k;
  a.nb = k / 32;
  return a;
}

// Packed weight row views.
struct WeightView {
  const uint8_t* base;
  int64_t row_bytes;
  int64_t hdr_bytes;
  __device__ __forceinline__ const uint8_t* row(int64_t n) const { return base + n * row_bytes; }
};

}  // namespace qblk
