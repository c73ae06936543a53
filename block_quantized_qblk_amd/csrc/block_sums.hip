// Test export: the integer block sums S[m][n][j] that the products scale and
// accumulate, computed with the same unpack and dot helpers as qblk_gemv
// (wmrh.cn "bare engine" article, §2.2: integer multiply-add inside each
// block). Q4_0 sums are over (nibble - 8) * code, Q8_0 over code * code and
// Q4_K over nibble * code. One thread per (m, n, j); small shapes only.
#include "qblk_device.h"

namespace qblk {
namespace {

template <int TYPE>
__global__ __launch_bounds__(256) void block_sums_kernel(WeightView W, int64_t n, int64_t nb,
                                                         ActView A, int64_t m,
                                                         int32_t* __restrict__ out) {
  const int64_t gid = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (gid >= m * n * nb) return;
  const int64_t blk = gid % nb;
  const int64_t nn = (gid / nb) % n;
  const int64_t mm = gid / (nb * n);
  const uint8_t* wquant = W.row(nn) + W.hdr_bytes;
  const uint8_t* ap = A.codes(mm, blk);
  const uint4 a0 = load16(ap);
  const uint4 a1 = load16(ap + 16);
  int S;
  if constexpr (TYPE == kQ8_0) {
    S = dot_i8x32(load16(wquant + 32 * blk), load16(wquant + 32 * blk + 16), a0, a1);
  } else {
    S = dot_nib32(load16(wquant + 16 * blk), a0, a1);
    if constexpr (TYPE == kQ4_0 || TYPE == kQ4_0H) S -= 8 * __float_as_int(A.dsum(mm, blk).y);
  }
  out[gid] = S;
}

}  // namespace

hipError_t launch_block_sums(int type, const void* wq, int64_t n, int64_t k, const void* xq,
                             int64_t m, int32_t* sums, hipStream_t s) {
  WeightView W;
  W.base = static_cast<const uint8_t*>(wq);
  W.row_bytes = row_bytes(type, k);
  W.hdr_bytes = header_bytes(type, k);
  const ActView A = make_act(xq, m, k);
  const int64_t nb = k / 32;
  const int64_t grid = (m * n * nb + 255) / 256;
  const dim3 g(static_cast<uint32_t>(grid));
  switch (type) {
    case kQ4_0: hipLaunchKernelGGL(block_sums_kernel<kQ4_0>, g, dim3(256), 0, s, W, n, nb, A, m, sums); break;
    case kQ8_0: hipLaunchKernelGGL(block_sums_kernel<kQ8_0>, g, dim3(256), 0, s, W, n, nb, A, m, sums); break;
    case kQ4_0H: hipLaunchKernelGGL(block_sums_kernel<kQ4_0H>, g, dim3(256), 0, s, W, n, nb, A, m, sums); break;
    default: hipLaunchKernelGGL(block_sums_kernel<kQ4_K>, g, dim3(256), 0, s, W, n, nb, A, m, sums); break;
  }
  return hipGetLastError();
}

}  // namespace qblk
