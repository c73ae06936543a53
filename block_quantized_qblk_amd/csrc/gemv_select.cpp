// Host-side choice of the GEMV kernel instance for a product's shape. Pure
// host C++ (no HIP device code), shared by the launchers in gemv.hip and the
// introspection export qblk_gemv_variant.
#include <stdio.h>

#include "qblk_internal.h"

namespace qblk {

// Kernel variant per shape, from measurements on MI355X over the 7B- and
// 70B-shaped Q4_K matrices (graphs of back-to-back launches): at batch 1 the
// classic kernel with 4 rows per wave streams the largest matrices best
// (6.0-6.5 TB/s; the 7B-shaped gate/up, 28672 x 4096, with the in-launch
// handoff 13.9 against 16.5 us with 2 rows), with 2 rows per wave the
// mid-size ones (activations staged in LDS), 1 row per wave with 2 chunks in
// flight the small ones; at batch
// 2-8, 8 rows per wave above 16k rows and 4 above 3k (70B layer at batch 4:
// 142 us against 179 us with 2 rows per wave). All variants give
// bit-identical results.
GemvVariant select_gemv(int type, int64_t n, int64_t k, int b, int mode) {
  GemvVariant v{};
  v.type = type;
  v.b = b;
  v.waves = 4;
  v.sync = mode == kGemvInLaunch;
  v.fused = mode == kGemvLdsFused;
  const int64_t nb = k / 32;
  // Q4_K at 2-8 activation rows with whole 2048-element chunks: the
  // matrix-core kernel with the direct-load LDS ring (gemv_ring_kernel).
  // Measured against the dot4 kernels with the in-launch quantization, it is
  // faster on every 70B-, 7B- and shard-shaped matrix at 2 to 8 rows (at 2
  // rows: 70B gate/up 44.7-47.1 against 49.5-49.9 us, down 24.9 against 27.2,
  // o 10.5 against 11.7, 7B down 11.4 against 16.0; at 8 rows: gate/up 69-72
  // against 92-94 us, down 34 against 48, q/k/v 19.5 against 28.0).
  // With more 16-row tiles than the two-per-CU grid holds and at least two
  // chunks per tile, a fixed grid walks them (gemv_ring_tiles_kernel), so
  // that each tile's first chunk loads while the last one's is computed: 70B
  // gate/up with the in-launch quantization 50-52 against 56 us at 4 rows, 48
  // against 55 at 3, q/k/v (640 tiles) 14.9 against 15.4 us; at 512 tiles or
  // fewer (70B o and down) the one-tile kernel stays faster (o 10.9 against
  // 11.3 us).
  if (type == kQ4_K && b >= 2 && b <= 8 && k % 2048 == 0) {
    v.ring = true;
    v.ring_tiles = (n + 15) / 16 > kRingGrid && k >= 4096;
    return v;
  }
  if (mode == kGemvLdsFused) {
    v.pipe = true;
    v.r = n >= 8192 ? 4 : 2;
    v.u = 1;
    v.alds = false;
    return v;
  }
  v.pipe = false;
  v.alds = gemv_stage_acts_in_lds(b, nb);
  auto set = [&](int r, int u) {
    v.r = r;
    v.u = u;
    return v;
  };
  if (b == 1) {
    if (n >= 16384) return set(4, 1);
    if (n >= 8192 && k >= 16384) return set(4, 1);
    // long rows of a mid-size matrix with the in-launch handoff: two chunks
    // per step (7B-shaped down, 4096 x 14336: 10.5 against 11.2 us; with a
    // quantized activation one chunk stays faster, 9.7 against 10.8 us)
    if (v.sync && n >= 3072 && n < 8192 && k >= 8192) return set(2, 2);
    // Q4_0 / Q8_0 rows (no super-block headers, fewer instructions per
    // block) on a quantized activation: two chunks per step (Q4_0 4096 x
    // 14336: 8.3 against 9.0 us; 4096 x 4096: 4.2 against 4.3 us; Q8_0
    // 14336 x 4096: 13.2-14.1 against 14.2 us in two runs; Q4_K is slower
    // this way on the 7B-shaped q/k/v and down)
    if (mode == kGemvQuantized && type != kQ4_K && n >= 3072) return set(2, 2);
    if (n >= 3072) return set(2, 1);
    return set(1, 2);
  }
  // several activation rows: every row a wave owns re-uses the activation
  // registers, and at batch 2-8 those re-reads bound the kernel, so the
  // larger matrices take more rows per wave
  if (n >= 16384) return set(8, 1);
  if (n >= 3072) {
    // long rows at batch 4 and above: 8 rows per wave (70B-shaped down,
    // 8192 x 28672: 36.8 against 37.8 us at batch 4, 48.6 against 53.2 at
    // 8; slower at batch 2); short rows: 2 (7B-shaped q/k/v, 6144 x 4096:
    // 9.6 against 9.7 us at batch 4, 13.6 against 14.7 at 8)
    if (b >= 4 && k >= 16384) return set(8, 1);
    if (k <= 4096) return set(2, 1);
    // Q4_K, 6k-8k rows of 8k weights: 8-wave workgroups, one per compute
    // unit, so each CU stages the activation rows once instead of twice
    // (70B-shaped o, 8192 x 8192, in-launch handoff: 11.7 against 13.0 us
    // at batch 2, 13.2 against 15.6 at 4, 20.3 against 21.4 at 8; with
    // 10240 rows, 320 such workgroups on 256 CUs, slower: 18.5 against 18.2
    // at batch 4)
    if (type == kQ4_K && n > 6144 && n <= 8192 && k <= 8192) v.waves = 8;
    return set(4, 1);
  }
  return set(1, 1);
}

// qblk_gemm with at most 8 activation rows: the decode GEMV kernels stream
// the weights faster than the few-rows GEMM, whose grid has one workgroup
// per 64 weight rows. Measured (quantized activation, GEMM against GEMV):
// at 1-4 rows on every type and shape (Q4_K 4096 x 14336 at 1 row 30.6
// against 9.6 us, Q8_0 14336 x 4096 at 4 rows 20.1 against 18.7 us); at 8
// rows with up to 8192 weight rows (Q4_0 4096 x 4096 14.1 against 7.7 us)
// and wherever the matrix-core GEMV runs (Q4_K 14336 x 4096 13.5 against
// 12.9 us), but not for Q4_0 / Q8_0 with 14336 rows (Q8_0 20.8 against 24.0).
bool gemm_runs_gemv(int type, int64_t n, int64_t k, int64_t m) {
  if (m > 8) return false;
  if (m <= 4 || n <= 8192) return true;
  return select_gemv(type, n, k, static_cast<int>(m), kGemvQuantized).ring;
}

int gemv_variant_name(const GemvVariant& v, char* buf, size_t len) {
  const char* t = v.sync ? "true" : "false";
  const char* a = v.alds ? "true" : "false";
  if (v.ring) return snprintf(buf, len, "%s<%d, %s>", v.ring_tiles ? "gemv_ring_tiles_kernel" : "gemv_ring_kernel", v.b, t);
  if (v.pipe)
    return snprintf(buf, len, "gemv_pipe_kernel<%d, %d, %d, %s, %s, %s>", v.type, v.b, v.r,
                    v.fused ? "true" : "false", t, a);
  // every template argument, the waves per workgroup included, as the
  // kernel's name reads in a profiler's trace
  return snprintf(buf, len, "gemv_kernel<%d, %d, %d, %d, %s, %s, %d>", v.type, v.b, v.r, v.u, t, a, v.waves);
}

}  // namespace qblk
