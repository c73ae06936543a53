// C-ABI front end: argument validation, then one launch on the caller's
// stream. Nothing is enqueued when validation fails. No allocation, no
// synchronization, no state except a thread-local last HIP error.
#include <hip/hip_runtime_api.h>

#include "../../include/qblk.h"
#include "qblk_internal.h"

#define QBLK_EXPORT extern "C" __attribute__((visibility("default")))

namespace {

thread_local int g_last_hip_error = 0;
// the in-launch handoff's wait bound for launches from this thread (a test
// setting; qblk_gemv_f32_set_wait_limit)
thread_local int64_t g_wait_ticks = qblk::kGemvWaitTicks;

bool valid_type(int t) {
  return t == QBLK_Q4_0 || t == QBLK_Q8_0 || t == QBLK_Q4_K || t == QBLK_Q4_0_F16;
}

// Largest k accepted: row offsets inside the kernels are 32-bit.
constexpr int64_t kMaxGemmK = int64_t(1) << 24;
constexpr int64_t kMaxK = int64_t{1} << 28;

bool valid_k(int t, int64_t k) {
  if (k <= 0 || k > kMaxK) return false;
  return t == QBLK_Q4_K ? (k % 256 == 0) : (k % 32 == 0);
}

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

// a * b <= lim for a, b >= 0, decided without forming the product (sizes
// come from the caller and may be arbitrarily large)
bool mul_within(int64_t a, int64_t b, int64_t lim) { return a == 0 || b <= lim / a; }
constexpr int64_t kMaxBytes = INT64_MAX;

// A dispatch holds fewer than 2^32 work-items per grid dimension.
constexpr int64_t kMaxGridThreads = (int64_t{1} << 32) - 256;

static_assert(QBLK_GEMV_MULTI_MAX == qblk::kGemvMultiMax, "descriptor list sizes agree");
static_assert(QBLK_NOALLOC_MAX_K == qblk::kNoallocMaxK && QBLK_NOALLOC_MAX_ACT_BYTES == qblk::kNoallocMaxActBytes,
              "allocation-free limits agree");

qblk_status finish(hipError_t e) {
  if (e != hipSuccess) {
    g_last_hip_error = static_cast<int>(e);
    return QBLK_ERR_LAUNCH;
  }
  return QBLK_OK;
}

// Shared validation of the product entry points.
qblk_status check_product(int type, const void* wq, int64_t n, int64_t k, const void* xq, int64_t m,
                  const void* out, int64_t ldy) {
  if (!valid_type(type)) return QBLK_ERR_ARG;
  if (n < 0 || m < 0) return QBLK_ERR_ARG;
  if (!valid_k(type, k)) return QBLK_ERR_SHAPE;
  if (n == 0 || m == 0) return QBLK_OK;
  if (wq == nullptr || xq == nullptr || out == nullptr) return QBLK_ERR_ARG;
  if (ldy < n) return QBLK_ERR_SHAPE;
  if (!aligned(wq, 16) || !aligned(xq, 16) || !aligned(out, 4)) return QBLK_ERR_ALIGN;
  return QBLK_OK;
}

}  // namespace

QBLK_EXPORT int qblk_abi_version(void) { return QBLK_VERSION; }

QBLK_EXPORT const char* qblk_strerror(int status) {
  switch (status) {
    case QBLK_OK: return "ok";
    case QBLK_ERR_ARG: return "invalid argument (null pointer, negative size or unknown type)";
    case QBLK_ERR_SHAPE: return "invalid shape (k not a positive multiple of the block size, or leading dimension too small)";
    case QBLK_ERR_ALIGN: return "misaligned pointer or leading dimension";
    case QBLK_ERR_UNSUPPORTED: return "size not supported by this entry point";
    case QBLK_ERR_LAUNCH: return "HIP launch failed (see qblk_last_hip_error)";
    default: return "unknown status";
  }
}

QBLK_EXPORT int qblk_last_hip_error(void) { return g_last_hip_error; }

QBLK_EXPORT size_t qblk_weight_row_bytes(int type, int64_t k) {
  if (!valid_type(type) || !valid_k(type, k)) return 0;
  return static_cast<size_t>(qblk::row_bytes(type, k));
}

QBLK_EXPORT size_t qblk_weight_bytes(int type, int64_t n, int64_t k) {
  const int64_t rb = static_cast<int64_t>(qblk_weight_row_bytes(type, k));
  if (n < 0 || !mul_within(n, rb, kMaxBytes)) return 0;
  return static_cast<size_t>(n * rb);
}

QBLK_EXPORT size_t qblk_act_bytes(int64_t m, int64_t k) {
  if (m < 0 || k <= 0 || k % 32 != 0 || !mul_within(m, k, kMaxBytes / 2)) return 0;
  return static_cast<size_t>(m * k + 8 * m * (k / 32));
}

QBLK_EXPORT qblk_status qblk_pack_weights(int type, const float* w, int64_t n, int64_t k, int64_t ldw,
                                  void* wq, hipStream_t stream) {
  if (!valid_type(type) || n < 0) return QBLK_ERR_ARG;
  if (!valid_k(type, k)) return QBLK_ERR_SHAPE;
  if (n == 0) return QBLK_OK;
  if (w == nullptr || wq == nullptr) return QBLK_ERR_ARG;
  if (ldw < k) return QBLK_ERR_SHAPE;
  if (!aligned(w, 16) || ldw % 4 != 0 || !aligned(wq, 16)) return QBLK_ERR_ALIGN;
  if (!mul_within(n, k / 32, kMaxGridThreads / 8)) return QBLK_ERR_UNSUPPORTED;
  (void)hipGetLastError();
  return finish(qblk::launch_pack_weights(type, w, n, k, ldw, wq, qblk::row_bytes(type, k), stream));
}

QBLK_EXPORT qblk_status qblk_quantize_act(const float* x, int64_t m, int64_t k, int64_t ldx, void* xq,
                                  hipStream_t stream) {
  if (m < 0) return QBLK_ERR_ARG;
  if (k <= 0 || k % 32 != 0) return QBLK_ERR_SHAPE;
  if (m == 0) return QBLK_OK;
  if (x == nullptr || xq == nullptr) return QBLK_ERR_ARG;
  if (ldx < k) return QBLK_ERR_SHAPE;
  if (!aligned(x, 16) || ldx % 4 != 0 || !aligned(xq, 16)) return QBLK_ERR_ALIGN;
  if (!mul_within(m, k / 32, kMaxGridThreads / 4)) return QBLK_ERR_UNSUPPORTED;
  (void)hipGetLastError();
  return finish(qblk::launch_quantize_act(x, m, k, ldx, xq, stream));
}

QBLK_EXPORT qblk_status qblk_gemv(int type, const void* wq, int64_t n, int64_t k, const void* xq,
                          int64_t batch, float* y, int64_t ldy, hipStream_t stream) {
  const qblk_status st = check_product(type, wq, n, k, xq, batch, y, ldy);
  if (st != QBLK_OK || n == 0 || batch == 0) return st;
  if (batch > QBLK_GEMV_MAX_BATCH) return QBLK_ERR_UNSUPPORTED;
  if (n > kMaxGridThreads / 64) return QBLK_ERR_UNSUPPORTED;
  (void)hipGetLastError();
  return finish(qblk::launch_gemv(type, wq, n, k, xq, batch, y, ldy, stream));
}

QBLK_EXPORT int qblk_gemv_f32_max_batch(int64_t k) {
  if (k <= 0 || k % 32 != 0 || k > kMaxK) return 0;
  return static_cast<int>(qblk::gemv_f32_max_batch(k));
}

QBLK_EXPORT size_t qblk_gemv_f32_work_bytes(int64_t batch, int64_t k) {
  if (batch < 0 || k <= 0 || k % 32 != 0 || k > kMaxK || batch > qblk::gemv_f32_max_batch(k))
    return 0;
  return static_cast<size_t>(qblk::gemv_f32_work_bytes(batch, k));
}

QBLK_EXPORT qblk_status qblk_gemv_f32(int type, const void* wq, int64_t n, int64_t k, const float* x,
                              int64_t ldx, int64_t batch, float* y, int64_t ldy, void* work,
                              hipStream_t stream) {
  const qblk_status st = check_product(type, wq, n, k, x, batch, y, ldy);
  if (st != QBLK_OK || n == 0 || batch == 0) return st;
  if (work == nullptr) return QBLK_ERR_ARG;
  if (ldx < k) return QBLK_ERR_SHAPE;
  if (!aligned(x, 16) || ldx % 4 != 0 || !aligned(work, 256)) return QBLK_ERR_ALIGN;
  if (batch > qblk::gemv_f32_max_batch(k)) return QBLK_ERR_UNSUPPORTED;
  if (n > kMaxGridThreads / 64) return QBLK_ERR_UNSUPPORTED;
  (void)hipGetLastError();
  return finish(qblk::launch_gemv_f32(type, wq, n, k, x, ldx, batch, y, ldy,
                                      qblk::gemv_work_in(work, batch, k), g_wait_ticks, stream));
}

QBLK_EXPORT qblk_status qblk_gemv_f32_noalloc(int type, const void* wq, int64_t n, int64_t k,
                                              const float* x, int64_t ldx, int64_t batch, float* y,
                                              int64_t ldy, hipStream_t stream) {
  const qblk_status st = check_product(type, wq, n, k, x, batch, y, ldy);
  if (st != QBLK_OK || n == 0 || batch == 0) return st;
  if (ldx < k) return QBLK_ERR_SHAPE;
  if (!aligned(x, 16) || ldx % 4 != 0) return QBLK_ERR_ALIGN;
  if (batch > qblk::gemv_f32_max_batch(k) || k > qblk::kNoallocMaxK ||
      static_cast<int64_t>(qblk_act_bytes(batch, k)) > qblk::kNoallocMaxActBytes)
    return QBLK_ERR_UNSUPPORTED;
  if (n > kMaxGridThreads / 64) return QBLK_ERR_UNSUPPORTED;
  qblk::GemvWork w{};
  const hipError_t e = qblk::gemv_scratch_work(stream, &w);
  if (e == hipErrorInvalidDevice) return QBLK_ERR_ARG;
  if (e != hipSuccess) return finish(e);
  (void)hipGetLastError();
  return finish(qblk::launch_gemv_f32(type, wq, n, k, x, ldx, batch, y, ldy, w, g_wait_ticks, stream));
}

QBLK_EXPORT size_t qblk_gemv_f32_fallback_offset(int64_t batch, int64_t k) {
  if (qblk_gemv_f32_work_bytes(batch, k) == 0 || batch == 0) return 0;
  return static_cast<size_t>(qblk::gemv_fallback_offset(batch, k));
}

QBLK_EXPORT qblk_status qblk_gemv_f32_set_wait_limit(int64_t ticks) {
  g_wait_ticks = ticks < 0 ? qblk::kGemvWaitTicks : ticks;
  return QBLK_OK;
}

QBLK_EXPORT qblk_status qblk_gemv_variant(int type, int64_t n, int64_t k, int64_t batch, int fused,
                                  char* name, size_t len) {
  if (!valid_type(type) || n <= 0 || batch <= 0 || name == nullptr || len == 0) return QBLK_ERR_ARG;
  if (!valid_k(type, k)) return QBLK_ERR_SHAPE;
  if (batch > (fused ? qblk::gemv_f32_max_batch(k) : QBLK_GEMV_MAX_BATCH)) return QBLK_ERR_UNSUPPORTED;
  const int b = static_cast<int>(batch < 8 ? batch : 8);
  const int mode = !fused ? qblk::kGemvQuantized
                          : (qblk::gemv_f32_lds_fused(n, k, batch) ? qblk::kGemvLdsFused : qblk::kGemvInLaunch);
  const int w = qblk::gemv_variant_name(qblk::select_gemv(type, n, k, b, mode), name, len);
  return w > 0 && static_cast<size_t>(w) < len ? QBLK_OK : QBLK_ERR_ARG;
}

QBLK_EXPORT qblk_status qblk_gemv_multi(int type, const qblk_gemv_desc* descs, int count, int64_t batch,
                                hipStream_t stream) {
  if (!valid_type(type) || count < 0 || batch < 0) return QBLK_ERR_ARG;
  if (count == 0 || batch == 0) return QBLK_OK;
  if (descs == nullptr) return QBLK_ERR_ARG;
  if (count > QBLK_GEMV_MULTI_MAX) return QBLK_ERR_UNSUPPORTED;
  int64_t wgs = 0;
  for (int i = 0; i < count; ++i) {
    const qblk_gemv_desc& d = descs[i];
    const qblk_status st = check_product(type, d.wq, d.n, d.k, d.xq, batch, d.y, d.ldy);
    if (st != QBLK_OK) return st;
    if (d.n > kMaxGridThreads) return QBLK_ERR_UNSUPPORTED;
    wgs += (d.n + 7) / 8;  // at most 2 rows per wave, 4 waves per workgroup
  }
  if (batch > QBLK_GEMV_MAX_BATCH) return QBLK_ERR_UNSUPPORTED;
  if (wgs > kMaxGridThreads / 256) return QBLK_ERR_UNSUPPORTED;
  qblk::GemvDesc d[QBLK_GEMV_MULTI_MAX];
  for (int i = 0; i < count; ++i)
    d[i] = qblk::GemvDesc{descs[i].wq, descs[i].n, descs[i].k, descs[i].xq, descs[i].y, descs[i].ldy};
  (void)hipGetLastError();
  return finish(qblk::launch_gemv_multi(type, d, count, batch, stream));
}

QBLK_EXPORT qblk_status qblk_gemv_float(int type, const void* wq, int64_t n, int64_t k, const float* x,
                                int64_t ldx, int64_t batch, float* y, int64_t ldy,
                                hipStream_t stream) {
  const qblk_status st = check_product(type, wq, n, k, x, batch, y, ldy);
  if (st != QBLK_OK || n == 0 || batch == 0) return st;
  if (ldx < k) return QBLK_ERR_SHAPE;
  if (ldx % 4 != 0) return QBLK_ERR_ALIGN;
  if (batch > QBLK_GEMV_MAX_BATCH) return QBLK_ERR_UNSUPPORTED;
  if (n > kMaxGridThreads / 64) return QBLK_ERR_UNSUPPORTED;
  (void)hipGetLastError();
  return finish(qblk::launch_gemv_float(type, wq, n, k, x, ldx, batch, y, ldy, stream));
}

QBLK_EXPORT qblk_status qblk_gemm(int type, const void* wq, int64_t n, int64_t k, const void* xq,
                          int64_t m, float* y, int64_t ldy, hipStream_t stream) {
  const qblk_status st = check_product(type, wq, n, k, xq, m, y, ldy);
  if (st != QBLK_OK || n == 0 || m == 0) return st;
  // grid: x = n / 128 workgroups of 256 work-items, y = m / 128 (<= 65535),
  // or, in the few-rows form, x = n / 16 at most and y = m / 64; a workgroup
  // addresses its activation and weight rows with 32-bit offsets, so k is
  // limited to 2^24
  const bool few = qblk::gemm_few_rows(n, m);
  const int64_t wgs = few ? (n + 15) / 16 : (n + 127) / 128;
  if (wgs > kMaxGridThreads / 256 || (m + 127) / 128 > 65535 || k > kMaxGemmK)
    return QBLK_ERR_UNSUPPORTED;
  (void)hipGetLastError();
  if (qblk::gemm_runs_gemv(type, n, k, m)) {  // few rows: the decode GEMV kernels
    if (n > kMaxGridThreads / 64) return QBLK_ERR_UNSUPPORTED;
    return finish(qblk::launch_gemv(type, wq, n, k, xq, m, y, ldy, stream));
  }
  return finish(qblk::launch_gemm(type, wq, n, k, xq, m, y, ldy, stream));
}

namespace {

bool valid_kv(int type, int64_t head_dim) {
  return (type == QBLK_Q4_0 || type == QBLK_Q8_0 || type == QBLK_Q4_0_F16) &&
         (head_dim == 64 || head_dim == 128 || head_dim == 256);
}

}  // namespace

QBLK_EXPORT size_t qblk_kv_cache_bytes(int type, int64_t n_kv, int64_t n_ctx, int64_t head_dim) {
  if (!valid_kv(type, head_dim) || n_kv <= 0 || n_ctx <= 0 || n_kv > 65535) return 0;
  const int64_t head_bytes = n_kv * qblk::row_bytes(type, head_dim);  // < 2^25
  if (!mul_within(n_ctx, head_bytes, kMaxBytes)) return 0;
  return static_cast<size_t>(n_ctx * head_bytes);
}

QBLK_EXPORT qblk_status qblk_kv_store(int type, const float* x, int64_t n_kv, int64_t head_dim, int64_t ldx,
                              void* cache, int64_t n_ctx, int64_t pos, hipStream_t stream) {
  if (!(type == QBLK_Q4_0 || type == QBLK_Q8_0 || type == QBLK_Q4_0_F16) || n_kv < 0) return QBLK_ERR_ARG;
  if (!valid_kv(type, head_dim) || n_ctx <= 0 || pos < 0 || pos >= n_ctx) return QBLK_ERR_SHAPE;
  if (n_kv == 0) return QBLK_OK;
  if (x == nullptr || cache == nullptr) return QBLK_ERR_ARG;
  if (ldx < head_dim) return QBLK_ERR_SHAPE;
  if (!aligned(x, 16) || ldx % 4 != 0 || !aligned(cache, 16)) return QBLK_ERR_ALIGN;
  if (n_kv > 65535 || qblk_kv_cache_bytes(type, n_kv, n_ctx, head_dim) == 0) return QBLK_ERR_UNSUPPORTED;
  const int64_t rb = qblk::row_bytes(type, head_dim);
  (void)hipGetLastError();
  return finish(qblk::launch_pack_weights(type, x, n_kv, head_dim, ldx, static_cast<uint8_t*>(cache) + pos * rb,
                                          n_ctx * rb, stream));
}

QBLK_EXPORT qblk_status qblk_kv_scores(int type, const void* cache, int64_t n_kv, int64_t n_ctx, int64_t n_tok,
                               int64_t head_dim, const void* q, int64_t n_head, float* scores, int64_t lds,
                               hipStream_t stream) {
  if (!(type == QBLK_Q4_0 || type == QBLK_Q8_0 || type == QBLK_Q4_0_F16)) return QBLK_ERR_ARG;
  if (n_kv <= 0 || n_head <= 0 || n_head % n_kv != 0) return QBLK_ERR_ARG;
  if (!valid_kv(type, head_dim) || n_ctx <= 0 || n_tok < 0 || n_tok > n_ctx) return QBLK_ERR_SHAPE;
  if (n_tok == 0) return QBLK_OK;
  if (cache == nullptr || q == nullptr || scores == nullptr) return QBLK_ERR_ARG;
  if (lds < n_tok) return QBLK_ERR_SHAPE;
  if (!aligned(cache, 16) || !aligned(q, 16) || !aligned(scores, 4)) return QBLK_ERR_ALIGN;
  if (n_head / n_kv > 8 || n_kv > 65535 || qblk_kv_cache_bytes(type, n_kv, n_ctx, head_dim) == 0)
    return QBLK_ERR_UNSUPPORTED;
  (void)hipGetLastError();
  return finish(qblk::launch_kv_scores(type, cache, n_kv, n_ctx, n_tok, head_dim, q, n_head, scores, lds, stream));
}

QBLK_EXPORT qblk_status qblk_block_sums(int type, const void* wq, int64_t n, int64_t k, const void* xq,
                                int64_t m, int32_t* sums, hipStream_t stream) {
  const qblk_status st = check_product(type, wq, n, k, xq, m, sums, n);
  if (st != QBLK_OK || n == 0 || m == 0) return st;
  if (!mul_within(m, n, kMaxGridThreads) || !mul_within(m * n, k / 32, kMaxGridThreads))
    return QBLK_ERR_UNSUPPORTED;
  (void)hipGetLastError();
  return finish(qblk::launch_block_sums(type, wq, n, k, xq, m, sums, stream));
}
