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
  const Q8Group r = quantize_group8(e);

  *reinterpret_cast<uint2*>(xq + row * k + 32 * blk + 8 * sub) = r.codes;
  if (sub == 0) {
    float2 ds;
    ds.x = r.d;
    ds.y = __int_as_float(r.sum);
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
