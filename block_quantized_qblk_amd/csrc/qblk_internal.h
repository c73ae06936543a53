// Host-side declarations shared between the C-ABI front end (api.cpp) and
// the kernel translation units. Not part of the public ABI.
#pragma once

#include <hip/hip_runtime_api.h>
#include <stddef.h>
#include <stdint.h>

namespace qblk {

enum : int { kQ4_0 = 1, kQ8_0 = 2, kQ4_K = 3, kQ4_0H = 4 };  // kQ4_0H: fp16-scale Q4_0

inline int64_t pad16(int64_t v) { return (v + 15) / 16 * 16; }

// Header region bytes of one packed row (scales, padded to 16 B).
inline int64_t header_bytes(int type, int64_t k) {
  switch (type) {
    case kQ4_0:
    case kQ8_0: return pad16(4 * (k / 32));
    case kQ4_K: return 16 * (k / 256);
    case kQ4_0H: return pad16(2 * (k / 32));
    default: return 0;
  }
}

// Bytes of one packed row.
inline int64_t row_bytes(int type, int64_t k) {
  switch (type) {
    case kQ4_0: return header_bytes(type, k) + 16 * (k / 32);
    case kQ8_0: return header_bytes(type, k) + 32 * (k / 32);
    case kQ4_K: return header_bytes(type, k) + 128 * (k / 256);
    case kQ4_0H: return header_bytes(type, k) + 16 * (k / 32);
    default: return 0;
  }
}

// Launchers (validated arguments only). Each returns the hipError_t of the
// launch.
hipError_t launch_quantize_act(const float* x, int64_t m, int64_t k, int64_t ldx, void* xq,
                               hipStream_t s);
// out_stride: bytes between output rows (row_bytes(type, k) for a dense matrix)
hipError_t launch_pack_weights(int type, const float* w, int64_t n, int64_t k, int64_t ldw,
                               void* wq, int64_t out_stride, hipStream_t s);
// Quantized KV cache: rows (h, t) of n_kv x n_ctx rows of row_bytes(type, head_dim).
hipError_t launch_kv_scores(int type, const void* cache, int64_t n_kv, int64_t n_ctx, int64_t n_tok,
                            int64_t head_dim, const void* q, int64_t n_head, float* scores, int64_t lds,
                            hipStream_t s);
hipError_t launch_gemv(int type, const void* wq, int64_t n, int64_t k, const void* xq,
                       int64_t batch, float* y, int64_t ldy, hipStream_t s);
// Fused quantize + GEMV (fp32 activations): up to 8 activation rows per
// launch (the local-memory variant keeps two 64-block slices of their codes
// in LDS, 5 KiB per row, so the limit does not depend on k).
inline int64_t gemv_f32_max_batch(int64_t k) { return k > 0 ? 8 : 0; }
// Whether the fused GEMV quantizes the activation in every workgroup's local
// memory (small single-row products with short rows) rather than once per
// launch into the caller's workspace. Measured on MI355X (Q4_K, graphs of
// back-to-back launches): per-workgroup quantization wins at batch 1 for
// K <= 2048 (2048 x 2048: 3.3 against 4.4 us) and for K = 4096 up to 2048
// rows (1024 x 4096: 4.5 against 4.7 us); the handoff wins from 4096 x 4096
// (5.4 against 6.0 us), at K = 8192, and at every size with several rows
// (7B-shaped q/k/v at batch 4: 9.8 against 18.2 us).
inline bool gemv_f32_lds_fused(int64_t n, int64_t k, int64_t batch) {
  return batch == 1 && n * k <= (int64_t(32) << 20) && (k <= 2048 || (k <= 4096 && n <= 2048));
}
// Workspace of the in-launch quantization: the activation buffer (same
// layout as qblk_quantize_act's), then 8 copies of one u64 flag per (activation row,
// 64-block slice), each copy padded to whole 128-byte lines.
inline int64_t gemv_flag_stride(int64_t k) {  // one flag per (activation row, 64-block slice)
  return (gemv_f32_max_batch(k) * ((k / 32 + 63) / 64) + 15) / 16 * 16;
}
inline int64_t gemv_flags_offset(int64_t batch, int64_t k) {
  return (batch * k + 8 * batch * (k / 32) + 255) / 256 * 256;
}
// then one uint32 counter of handoff fallbacks (workgroups that stopped
// waiting for the producers and quantized the activation themselves), on a
// 256-byte line of its own
inline int64_t gemv_fallback_offset(int64_t batch, int64_t k) {
  return gemv_flags_offset(batch, k) + 8 * 8 * gemv_flag_stride(k);
}
inline int64_t gemv_f32_work_bytes(int64_t batch, int64_t k) { return gemv_fallback_offset(batch, k) + 256; }
// The handoff's bounded wait, in ticks of the 100 MHz realtime counter: 20 ms.
constexpr int64_t kGemvWaitTicks = 2000000;
// GEMV activation staging: a workgroup copies the activation rows into LDS,
// per row whole 2 KiB chunks (64 blocks of 32 codes), then the (d, sum)
// pairs of all rows. Staged when the copy fits 16 KiB for one activation row
// (70B-shaped down, 36 KiB: 26.9 us staged against 24.6 us read from L2) or
// 40 KiB for several (70B-shaped gate/up at batch 4: 59.8 against 62.1 us).
constexpr uint32_t act_lds_row(uint32_t nb) { return ((nb + 63u) >> 6) * 2048u; }
constexpr uint32_t act_lds_bytes(int b, uint32_t nb) {
  return static_cast<uint32_t>(b) * (act_lds_row(nb) + 8u * nb);
}
constexpr uint32_t kActLdsMax = 16384;
constexpr uint32_t kActLdsMaxBatch = 40960;
constexpr bool gemv_stage_acts_in_lds(int b, int64_t nb) {
  return act_lds_bytes(b, static_cast<uint32_t>(nb)) <= (b == 1 ? kActLdsMax : kActLdsMaxBatch);
}
// Which GEMV kernel instance a product runs (pure host logic, no GPU):
// gemv_kernel<type, b, r, u, sync, alds, waves>, gemv_pipe_kernel<type,
// b, r, fused, sync, alds>, gemv_ring_kernel<b, sync> or
// gemv_ring_tiles_kernel<b, sync>. mode: how the activation reaches the
// kernel.
enum : int { kGemvQuantized = 0, kGemvLdsFused = 1, kGemvInLaunch = 2 };
struct GemvVariant {
  int type;
  int b;      // activation rows of the launch (1..8)
  int r;      // weight rows per wave
  int u;      // chunks per step (classic kernel)
  bool pipe;  // gemv_pipe_kernel (else gemv_kernel)
  bool sync;  // activation quantized once per launch (in-launch handoff)
  bool alds;  // activation rows staged in LDS
  bool fused; // activation quantized in every workgroup's LDS
  int waves;  // waves per workgroup (classic kernel)
  bool ring;  // gemv_ring_kernel (Q4_K, 2-8 rows: matrix cores, direct-load LDS ring)
  bool ring_tiles;  // ... as gemv_ring_tiles_kernel, a fixed grid walking the 16-row tiles
};
// The tile-walking grid of the matrix-core GEMV (two workgroups per CU); used
// when the 16-row tiles outnumber it and a tile has at least two chunks.
constexpr int64_t kRingGrid = 512;
GemvVariant select_gemv(int type, int64_t n, int64_t k, int b, int mode);
// Whether qblk_gemm runs the decode GEMV kernels (at most 8 activation rows)
bool gemm_runs_gemv(int type, int64_t n, int64_t k, int64_t m);
int gemv_variant_name(const GemvVariant& v, char* buf, size_t len);
// Where the in-launch handoff keeps its data: the activation buffer
// (qblk_quantize_act layout, batch rows of k), the 8 flag copies of
// gemv_flag_stride(k) u64 each, and the fallback counter.
struct GemvWork {
  uint8_t* act;
  uint64_t* flags;
  uint32_t* fallbacks;
};
// ... inside a caller's workspace of gemv_f32_work_bytes(batch, k) bytes
inline GemvWork gemv_work_in(void* work, int64_t batch, int64_t k) {
  uint8_t* b = static_cast<uint8_t*>(work);
  return GemvWork{b, reinterpret_cast<uint64_t*>(b + gemv_flags_offset(batch, k)),
                  reinterpret_cast<uint32_t*>(b + gemv_fallback_offset(batch, k))};
}
// ... inside the library's fixed device array (the allocation-free entry
// point): flags from byte 0, the counter at kScratchFlagBytes - 256, the
// activation buffer from kScratchFlagBytes. The flag region holds 8 copies
// of gemv_flag_stride(k) u64 for k <= kNoallocMaxK.
constexpr int64_t kScratchBytes = int64_t(1) << 20;
constexpr int64_t kScratchFlagBytes = int64_t(64) << 10;
constexpr int64_t kNoallocMaxActBytes = kScratchBytes - kScratchFlagBytes;  // 983040
constexpr int64_t kNoallocMaxK = int64_t(1) << 17;
static_assert(8 * 8 * ((8 * ((kNoallocMaxK / 32 + 63) / 64) + 15) / 16 * 16) <= kScratchFlagBytes - 256,
              "flag copies fit the flag region");
// The fixed array's GemvWork on the current device, after checking that
// `stream` belongs to it (hipErrorInvalidDevice if not). The array's address
// is looked up once per device, on the first call made there.
hipError_t gemv_scratch_work(hipStream_t stream, GemvWork* w);
// wait_ticks: the handoff's wait bound (kGemvWaitTicks outside tests)
hipError_t launch_gemv_f32(int type, const void* wq, int64_t n, int64_t k, const float* x,
                           int64_t ldx, int64_t batch, float* y, int64_t ldy, const GemvWork& work,
                           int64_t wait_ticks, hipStream_t s);
// one product of a multi-product GEMV launch (quantized activations)
struct GemvDesc {
  const void* wq;
  int64_t n;
  int64_t k;
  const void* xq;
  float* y;
  int64_t ldy;
};
constexpr int kGemvMultiMax = 16;
hipError_t launch_gemv_multi(int type, const GemvDesc* d, int count, int64_t batch, hipStream_t s);
hipError_t launch_gemv_float(int type, const void* wq, int64_t n, int64_t k, const float* x,
                             int64_t ldx, int64_t batch, float* y, int64_t ldy, hipStream_t s);
hipError_t launch_gemm(int type, const void* wq, int64_t n, int64_t k, const void* xq,
                       int64_t m, float* y, int64_t ldy, hipStream_t s);
// rows at or below which launch_gemm always takes the few-rows form
constexpr int64_t kGemmSmallMaxRows = 64;
// Whether launch_gemm takes the few-rows form (in 64-row chunks above 64
// rows). The 128 x 128 kernel's time is about one workgroup's while its grid
// holds at most one workgroup per CU, so on short matrices a few hundred rows
// run faster as chunks of the few-rows kernel. Measured (Q4_K, main against
// few-rows kernel): 4096 x 4096 at m = 256 91.0 against 57.0 us, 8192 x 8192
// at 256 176.9 against 119.9, 14336 x 4096 at 128 91.8 against 64.3 (at 256
// 92.7 against 121.7), 28672 x 4096 at 96 93.6 against 119.7; Q8_0 alike.
inline bool gemm_few_rows(int64_t n, int64_t m) {
  return m <= kGemmSmallMaxRows || (n <= 8192 && m <= 256) || (n <= 16384 && m <= 128);
}
// Whether the 128 x 128 kernel splits K over two groups of four waves: when
// its grid holds at most one workgroup per CU (256), and K has at least two
// steps of 128.
inline bool gemm_split_k(int64_t n, int64_t k, int64_t m) {
  return ((n + 127) / 128) * ((m + 127) / 128) <= 256 && k >= 256;
}
hipError_t launch_gemm_small(int type, const void* wq, int64_t n, int64_t k, const void* xq,
                             int64_t m, float* y, int64_t ldy, hipStream_t s);
hipError_t launch_block_sums(int type, const void* wq, int64_t n, int64_t k, const void* xq,
                             int64_t m, int32_t* sums, hipStream_t s);

}  // namespace qblk
