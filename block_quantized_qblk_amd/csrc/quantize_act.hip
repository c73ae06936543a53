// On-the-fly activation quantization to int8 32-blocks.
//
// "llama.cpp 推理引擎", §5.1 (symmetric quantization) at b = 8, applied per row
// and per 32 consecutive elements: d = max|x| / 127, q = round(x / d). Both
// divisions are IEEE fp32 divisions (correctly rounded) and round() is half
// away from zero, so the codes are bit-identical to any other correct
// implementation of the same rule. The block's integer code sum is stored
// beside d because the Q4_0 (nibble - 8) and Q4_K (min term) products need
// it.
#include "qblk_device.h"

#pragma clang fp contract(off)

namespace qblk {
namespace {

// Pack 8 int8 codes as two dwords in the element order 0,2,4,6 | 1,3,5,7.
__device__ __forceinline__ uint2 pack_group8(const int (&q)[8]) {
  uint2 r;
  r.x = (q[0] & 255u) | (q[2] & 255u) << 8 | (q[4] & 255u) << 16 | (q[6] & 255u) << 24;
  r.y = (q[1] & 255u) | (q[3] & 255u) << 8 | (q[5] & 255u) << 16 | (q[7] & 255u) << 24;
  return r;
}

// Four consecutive lanes handle one 32-block, 8 elements each.
__global__ __launch_bounds__(256) void quantize_act_kernel(const float* __restrict__ x, int64_t m,
                                                           int64_t k, int64_t ldx,
                                                           uint8_t* __restrict__ xq) {
  const int64_t nb = k / 32;
  const int64_t gid = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  const int64_t blk_all = gid >> 2;
  if (blk_all >= m * nb) return;  // a whole 4-lane group leaves together
  const int sub = static_cast<int>(gid & 3);
  const int64_t row = blk_all / nb;
  const int64_t blk = blk_all - row * nb;

  const float* src = x + row * ldx + 32 * blk + 8 * sub;
  const float4 v0 = *reinterpret_cast<const float4*>(src);
  const float4 v1 = *reinterpret_cast<const float4*>(src + 4);
  const float e[8] = {v0.x, v0.y, v0.z, v0.w, v1.x, v1.y, v1.z, v1.w};

  float amax = 0.0f;
#pragma unroll
  for (int i = 0; i < 8; ++i) amax = fmaxf(amax, fabsf(e[i]));
  amax = fmaxf(amax, __shfl_xor(amax, 1, 64));
  amax = fmaxf(amax, __shfl_xor(amax, 2, 64));

  const float d = __fdiv_rn(amax, 127.0f);
  int q[8];
  int s = 0;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    int qi = 0;
    if (d != 0.0f) {
      float r = roundf(__fdiv_rn(e[i], d));  // half away from zero
      r = fminf(fmaxf(r, -127.0f), 127.0f);
      qi = static_cast<int>(r);
    }
    q[i] = qi;
    s += qi;
  }
  s += __shfl_xor(s, 1, 64);
  s += __shfl_xor(s, 2, 64);

  *reinterpret_cast<uint2*>(xq + row * k + 32 * blk + 8 * sub) = pack_group8(q);
  if (sub == 0) {
    float2 ds;
    ds.x = d;
    ds.y = __int_as_float(s);
    *reinterpret_cast<float2*>(xq + m * k + 8 * (row * nb + blk)) = ds;
  }
}

}  // namespace

hipError_t launch_quantize_act(const float* x, int64_t m, int64_t k, int64_t ldx, void* xq,
                               hipStream_t s) {
  const int64_t threads = 4 * m * (k / 32);
  const int64_t grid = (threads + 255) / 256;
  hipLaunchKernelGGL(quantize_act_kernel, dim3(static_cast<uint32_t>(grid)), dim3(256), 0, s, x,
                     m, k, ldx, static_cast<uint8_t*>(xq));
  return hipGetLastError();
}

}  // namespace qblk
