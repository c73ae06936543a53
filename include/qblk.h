/*
 * qblk.h — C ABI of the block-quantized weight x activation product for
 * MI355X (gfx950).
 *
 * What is computed (pages cited by title and section):
 *   - Weights are quantized in 32-element blocks with one scale per block
 *     ("llama.cpp 推理引擎", §5.1 symmetric quantization, §5.3 Q4_0, §5.4 Q8_0)
 *     or in 256-element super-blocks of 8 sub-blocks with per-sub-block scale
 *     and min codes under fp16 super-block scales ("llama.cpp 推理引擎", §5.5
 *     K-quant; "llama.cpp：一个人、一个周末、一个改变 AI 推理格局的 C++ 文件",
 *     section 量化是怎么做到的？).
 *   - Activations are quantized on the fly to int8 32-blocks with an fp32
 *     scale (the §5.1 rule at 8 bits).
 *   - Inside each 32-block the dot product is integer (wmrh.cn "bare engine"
 *     article, §2.2: int4 x int8 multiply-add); the scales are applied
 *     outside it in fp32 ("llama.cpp 推理引擎", §6.4).
 *
 * Conventions shared by every entry point:
 *   - Pointers named w, x, y, wq, xq, sums are DEVICE pointers owned by the
 *     caller. The library never allocates, frees or synchronizes. Between
 *     calls it keeps only a thread-local last HIP error code, the
 *     thread-local handoff wait bound (qblk_gemv_f32_set_wait_limit), and,
 *     for qblk_gemv_f32_noalloc, a fixed device array per GPU with its
 *     address.
 *   - Work is enqueued on `stream` (NULL = the default stream) and the call
 *     returns without waiting. Calls are reentrant and thread-safe.
 *   - Every argument is validated BEFORE anything is enqueued; on any error
 *     nothing is enqueued and a negative qblk_status is returned (0 =
 *     success, negative = failure, the convention of the decode call on the
 *     page "【AI】端侧模型部署llama.cpp篇", section llama_decode).
 *   - Sizes are element counts (int64_t). m, n or batch equal to 0 is a valid
 *     empty call that enqueues nothing and returns QBLK_OK. Negative sizes are
 *     QBLK_ERR_ARG.
 *   - Buffers must not overlap unless stated.
 *
 * Byte layouts (little-endian; nb = k/32, nsb = k/256; a "row" is one output
 * channel n of the weight matrix W[n][k]):
 *   Q4_0 row : [fp32 d x nb, zero-padded to a multiple of 16 B]
 *              [16 B x nb: byte t of block b = (q[32b+2t]+8) | (q[32b+2t+1]+8) << 4]
 *              codes q in [-7, 7] when packed by this library; any nibble
 *              0..15 decodes as nibble - 8.
 *   Q4_0_F16 row: [fp16 d x nb, zero-padded to a multiple of 16 B]
 *              [16 B x nb: the Q4_0 nibbles]
 *   Q8_0 row : [fp32 d x nb, zero-padded to a multiple of 16 B]
 *              [32 int8 x nb; inside a block each group of 8 codes is stored
 *               in the element order 0,2,4,6,1,3,5,7]
 *   Q4_K row : [16 B header x nsb][128 B x nsb]
 *              header = fp16 d, fp16 d_min (<= 0), 12 bytes holding a 96-bit
 *              little-endian field with sc_j at bits [6j, 6j+6) and mn_j at
 *              bits [48+6j, 48+6j+6), j = 0..7;
 *              sub-block j of a super-block is bytes [16j, 16j+16) of its 128,
 *              byte t = q[32j+2t] | q[32j+2t+1] << 4, q in 0..15;
 *              weight value = (d*sc_j)*q + d_min*mn_j.
 *   Rows are stored back to back; qblk_weight_row_bytes gives the stride.
 *   Activation buffer (m rows, opaque to callers but fixed):
 *              [m*k int8 codes, row-major; inside each 32-block the groups
 *               of 8 use the order 0,2,4,6,1,3,5,7]
 *              [m*nb pairs (fp32 scale d, int32 sum of the block's 32 codes)]
 *
 * Alignment: wq, xq and x must be 16-byte aligned and ldx a multiple of 4;
 * y, sums and w need 4-byte alignment (w 16-byte, ldw a multiple of 4).
 */
#ifndef QBLK_H
#define QBLK_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

/* ABI version: the entry points and their argument lists. Layout version:
 * the byte layouts above (packed weight rows, activation buffer, KV cache
 * rows), which the library fixes itself where the pages list only fields
 * ("llama.cpp 推理引擎", §5.3-§5.5). qblk_abi_version() returns both, as
 * QBLK_VERSION; a caller holding packed buffers checks the layout part. */
#define QBLK_ABI_VERSION 2
#define QBLK_LAYOUT_VERSION 1
#define QBLK_VERSION ((QBLK_ABI_VERSION << 8) | QBLK_LAYOUT_VERSION)
#define QBLK_VERSION_ABI(v) ((v) >> 8)
#define QBLK_VERSION_LAYOUT(v) ((v) & 0xFF)

typedef enum {
  QBLK_Q4_0 = 1, /* 32-blocks, 4-bit codes, fp32 scale: 20 B / 32 weights */
  QBLK_Q8_0 = 2, /* 32-blocks, int8 codes, fp32 scale: 36 B / 32 weights  */
  QBLK_Q4_K = 3, /* 256-element super-blocks, 144 B / 256 weights         */
  QBLK_Q4_0_F16 = 4 /* 32-blocks, 4-bit codes, fp16 scale: 18 B / 32 weights,
                       the pages' own Q4_0 block ("llama.cpp 推理引擎",
                       §5.3) */
} qblk_type;

typedef enum {
  QBLK_OK = 0,
  QBLK_ERR_ARG = -1,         /* null pointer, negative size, unknown type    */
  QBLK_ERR_SHAPE = -2,       /* k not a positive multiple of 32 (256 for
                                Q4_K), or a leading dimension too small      */
  QBLK_ERR_ALIGN = -3,       /* pointer or leading dimension misaligned      */
  QBLK_ERR_UNSUPPORTED = -4, /* size beyond what a kernel supports (e.g.
                                gemv batch > QBLK_GEMV_MAX_BATCH)            */
  QBLK_ERR_LAUNCH = -5       /* the HIP launch failed; see
                                qblk_last_hip_error()                        */
} qblk_status;

#define QBLK_GEMV_MAX_BATCH 64

/* QBLK_VERSION of the loaded library: (ABI version << 8) | layout version. */
int qblk_abi_version(void);

/* Human-readable text for a qblk_status value (static storage). */
const char *qblk_strerror(int status);

/* hipError_t of the last failed launch on the calling thread (0 if none). */
int qblk_last_hip_error(void);

/* Bytes of one packed weight row of k elements (0 if type or k is invalid). */
size_t qblk_weight_row_bytes(int type, int64_t k);

/* Bytes of a packed n x k weight matrix = n * qblk_weight_row_bytes (0 if
 * invalid). */
size_t qblk_weight_bytes(int type, int64_t n, int64_t k);

/* Bytes of the activation buffer for m rows of k elements (0 if invalid):
 * m*k + 8*m*(k/32). */
size_t qblk_act_bytes(int64_t m, int64_t k);

/*
 * Weight quantization and packing (setup step).
 * "llama.cpp 推理引擎" §5.1 (symmetric rule; Q4_0 at 4 bits with codes in
 * [-7, 7], Q8_0 at 8 bits), §5.2 + §5.5 (Q4_K: asymmetric sub-blocks under
 * fp16 super-block scales).
 *   w   : fp32 [n][ldw], row n holds the k weights of output channel n.
 *   wq  : out, qblk_weight_bytes(type, n, k) bytes, layout above.
 * Rounding is half away from zero. Q4_0/Q8_0 decisions are taken in fp32
 * with IEEE division. Q4_0_F16: d = fp16 nearest (ties to even) of the fp32
 * amax/7, saturating at 65504, and q = round(x / d) against that fp16 d.
 * Q4_K decisions in fp64:
 *   m_j  = max(0, -min of sub-block j); d_min = -(smallest fp16 h with
 *   63*h >= max_j m_j); mn_j = smallest code with mn_j*h >= m_j;
 *   t_j  = max of sub-block j + mn_j*h; d = smallest fp16 with
 *   945*d >= max_j t_j; sc_j = smallest code with 15*sc_j*d >= t_j;
 *   q = clamp(round((x + mn_j*h) / (sc_j*d)), 0, 15) (0 when sc_j*d == 0).
 * Inputs must be finite; a super-block whose range exceeds what fp16 d can
 * express saturates d at 65504.
 * Errors: QBLK_ERR_ARG (null, negative n, unknown type), QBLK_ERR_SHAPE
 * (k invalid, ldw < k), QBLK_ERR_ALIGN, QBLK_ERR_LAUNCH.
 */
qblk_status qblk_pack_weights(int type, const float *w, int64_t n, int64_t k,
                      int64_t ldw, void *wq, hipStream_t stream);

/*
 * On-the-fly activation quantization: "llama.cpp 推理引擎" §5.1 at 8 bits,
 * per row and per 32 consecutive elements: d = max|x| / 127 (IEEE fp32
 * division), q = round_half_away(x / d) (IEEE fp32 division), d == 0 gives
 * q == 0; the int32 sum of the 32 codes is stored beside d.
 * Inputs must be finite: a block holding an infinity or a NaN gets
 * unspecified codes and scale (the other blocks are quantized as usual).
 *   x  : fp32 [m][ldx].
 *   xq : out, qblk_act_bytes(m, k) bytes, layout above.
 * Errors: QBLK_ERR_ARG, QBLK_ERR_SHAPE (k % 32 != 0, k <= 0, ldx < k),
 * QBLK_ERR_ALIGN, QBLK_ERR_LAUNCH.
 */
qblk_status qblk_quantize_act(const float *x, int64_t m, int64_t k, int64_t ldx,
                      void *xq, hipStream_t stream);

/*
 * Decode-path product (few activation rows). The per-block integer dot with
 * the scales applied outside it is the pages' quantized dot kernel
 * ("llama.cpp 推理引擎", §6.4 ggml_vec_dot_q4_0; wmrh.cn "bare engine"
 * article, §2.2: the Q4_K x Q8 dot as int4 x int8 multiply-adds); Q4_K
 * scale and min per sub-block as in §5.5. For b < batch, n < n:
 *   y[b*ldy + n] = sum over 32-blocks j of
 *     Q4_0/Q8_0: dw[n][j] * dx[b][j] * S[b][n][j]
 *     Q4_K     : dx[b][j] * ((d*sc_j)[n] * S[b][n][j] + (d_min*mn_j)[n] * A[b][j])
 *   where S is the integer dot of block j's weight codes (Q4_0: nibble - 8,
 *   Q8_0: int8, Q4_K: nibble) with the activation codes, and A the
 *   activation block sum. Accumulation is fp32 in an unspecified order.
 *   wq : packed weights [n] rows of k;  xq : activation buffer of `batch`
 *   rows of k (from qblk_quantize_act);  y : fp32 [batch][ldy].
 * Errors: QBLK_ERR_ARG, QBLK_ERR_SHAPE (k invalid or above 2^28, ldy < n),
 * QBLK_ERR_ALIGN, QBLK_ERR_UNSUPPORTED (batch > QBLK_GEMV_MAX_BATCH),
 * QBLK_ERR_LAUNCH.
 */
qblk_status qblk_gemv(int type, const void *wq, int64_t n, int64_t k, const void *xq,
              int64_t batch, float *y, int64_t ldy, hipStream_t stream);

/*
 * Several independent decode-path products in one launch: a descriptor list
 * (e.g. the q, k and v projections of a layer kept as separate matrices, all
 * reading the same or different activations). Each descriptor is one
 * qblk_gemv with the shared type and batch:
 *   wq : packed weights [n] rows of k;  xq : activation buffer of `batch`
 *   rows of k;  y : fp32 [batch][ldy].
 * The descriptors are read on the host during the call (the array need not
 * outlive it); their outputs must not overlap. Results are bit-identical to
 * qblk_gemv on each descriptor, with one exception: a Q4_K list at 2 to 8
 * activation rows (per group of 8 rows) runs the matrix-core kernel only if
 * every descriptor's k is a multiple of 2048; otherwise those whose k is
 * (where qblk_gemv_variant names gemv_ring_kernel or gemv_ring_tiles_kernel)
 * get the same block products and scale steps summed in another fp32 order.
 * Descriptors with n == 0 are skipped.
 * Errors: QBLK_ERR_ARG (type, count < 0, null descs), the qblk_gemv errors of
 * any descriptor, QBLK_ERR_UNSUPPORTED (count > QBLK_GEMV_MULTI_MAX, batch >
 * QBLK_GEMV_MAX_BATCH).
 */
#define QBLK_GEMV_MULTI_MAX 16
typedef struct qblk_gemv_desc {
  const void *wq;
  int64_t n;
  int64_t k;
  const void *xq;
  float *y;
  int64_t ldy;
} qblk_gemv_desc;
qblk_status qblk_gemv_multi(int type, const qblk_gemv_desc *descs, int count, int64_t batch,
                    hipStream_t stream);

/*
 * Decode-path product with the activation quantization fused in: the same
 * result, bit for bit, as qblk_quantize_act(x) followed by qblk_gemv, in one
 * launch. The activation is quantized with the qblk_quantize_act rule
 * ("llama.cpp 推理引擎", §5.1 at 8 bits):
 *   - batch 1 with k <= 2048, or k <= 4096 and n <= 2048 (and at most 32M
 *     weights): every workgroup quantizes the fp32 row, 64 blocks at a time,
 *     into its local memory while it streams its weight rows (work is not
 *     touched);
 *   - otherwise: the first workgroups of the launch quantize the rows once
 *     into `work`, one 64-block slice of one row each, and publish each slice
 *     with a tag unique to the launch; the workgroups issue their first
 *     weight loads, then wait for the tags (a bounded wait: past about 20 ms
 *     a workgroup adds 1 to the workspace's fallback counter and quantizes
 *     the rows itself, so the result never depends on scheduling).
 *   x    : fp32 [batch][ldx];  other arguments as qblk_gemv.
 *   work : device workspace of qblk_gemv_f32_work_bytes(batch, k) bytes,
 *          256-byte aligned, owned by the caller. It holds no state that a
 *          later call depends on (it need not be cleared), but calls that
 *          may run at the same time must use different workspaces.
 * batch <= qblk_gemv_f32_max_batch(k) (8 for any valid k, 0 when k is
 * invalid).
 * Errors: as qblk_gemv, plus QBLK_ERR_SHAPE for ldx < k, QBLK_ERR_ARG for a
 * null work, QBLK_ERR_ALIGN for x, ldx or work, QBLK_ERR_UNSUPPORTED for
 * batch > qblk_gemv_f32_max_batch(k).
 */
int qblk_gemv_f32_max_batch(int64_t k);
size_t qblk_gemv_f32_work_bytes(int64_t batch, int64_t k); /* 0 if invalid */
/* Byte offset inside the workspace of a uint32 counter that every launch
 * with the in-launch handoff increments once per workgroup that stopped
 * waiting and quantized the activation itself (0 if batch or k is invalid).
 * The library never resets it: a caller that zeroes it once can read how
 * often the fallback ran. */
size_t qblk_gemv_f32_fallback_offset(int64_t batch, int64_t k);
/* Test setting: the handoff's wait bound, in ticks of the 100 MHz realtime
 * counter, for launches made later from the calling thread (thread-local;
 * a negative value restores the default of 2,000,000 = 20 ms). A bound of 0
 * makes every workgroup that finds a slice unpublished take the fallback at
 * once; results are identical either way. */
qblk_status qblk_gemv_f32_set_wait_limit(int64_t ticks);
qblk_status qblk_gemv_f32(int type, const void *wq, int64_t n, int64_t k, const float *x,
                  int64_t ldx, int64_t batch, float *y, int64_t ldy, void *work,
                  hipStream_t stream);

/*
 * qblk_gemv_f32 for callers that cannot allocate (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc): the same
 * result, bit for bit, with no workspace argument. The in-launch handoff
 * uses a fixed device array of the library instead (1 MiB, held by each GPU
 * the library runs on until the process ends; its address is looked up once
 * per device, on the first call made there, with hipGetSymbolAddress). The
 * call allocates and frees nothing.
 * Limits: batch <= 8, k <= QBLK_NOALLOC_MAX_K and qblk_act_bytes(batch, k)
 * <= QBLK_NOALLOC_MAX_ACT_BYTES (e.g. k <= 98304 at batch 8); beyond them
 * QBLK_ERR_UNSUPPORTED, nothing enqueued.
 * Every call on a GPU shares that GPU's array, which keeps the last call's
 * contents. Nothing in it has to be cleared between calls (the flags only
 * ever hold zero or earlier launches' tags, which never match a later one),
 * but calls that overlap on one GPU race on it: calls from several streams
 * or threads must be serialized by the caller.
 * `stream` must belong to the current device (else QBLK_ERR_ARG).
 * Errors: as qblk_gemv_f32, without the workspace ones.
 */
#define QBLK_NOALLOC_MAX_K 131072
#define QBLK_NOALLOC_MAX_ACT_BYTES 983040
qblk_status qblk_gemv_f32_noalloc(int type, const void *wq, int64_t n, int64_t k, const float *x,
                                  int64_t ldx, int64_t batch, float *y, int64_t ldy,
                                  hipStream_t stream);

/*
 * Introspection (host only, no GPU work): the name of the kernel instance
 * that qblk_gemv (fused == 0) or qblk_gemv_f32 (fused != 0) launches for
 * this shape, for the first group of up to 8 activation rows, as the
 * kernel's template arguments: "gemv_kernel<type, rows, rows per wave,
 * chunks per step, in-launch quantization, activations in LDS, waves per
 * workgroup>", "gemv_ring_kernel<rows, in-launch quantization>" (Q4_K with 2
 * to 8 rows and k a multiple of 2048: matrix cores; one 16-row tile per
 * workgroup), "gemv_ring_tiles_kernel<rows, in-launch quantization>" (the
 * same with more than 512 tiles and k >= 4096: a fixed grid walks them) or
 * "gemv_pipe_kernel<type, rows, rows per wave, per-workgroup quantization,
 * in-launch quantization, activations in LDS>". Written NUL-terminated into
 * name[len]. Lets a test check that the instances a workload runs are the
 * ones its parity cases cover.
 * Errors: QBLK_ERR_ARG (type, n <= 0, batch <= 0, null name, len too
 * small), QBLK_ERR_SHAPE (k invalid), QBLK_ERR_UNSUPPORTED (batch beyond
 * the entry point's limit).
 */
qblk_status qblk_gemv_variant(int type, int64_t n, int64_t k, int64_t batch, int fused, char *name,
                      size_t len);

/*
 * Decode-path product with fp32 activations and no activation quantization,
 * the form of the pages' scalar Q4_0 dot ("llama.cpp 推理引擎", §6.4: each
 * weight decoded in place and multiplied by a float activation; Q4_K
 * weights decoded as in §5.5): for b < batch, n < n,
 *   y[b*ldy + n] = sum_k w[n][k] * x[b*ldx + k]
 *   where w is the decoded weight: Q4_0 / Q4_0_F16 d*(nibble - 8), Q8_0 d*q,
 *   Q4_K (d*sc_j)*q + (d_min*mn_j)*1. Accumulation is fp32 in an unspecified
 *   (but fixed) order.
 *   wq : packed weights [n] rows of k;  x : fp32 [batch][ldx], 16-byte
 *   aligned, ldx a multiple of 4;  y : fp32 [batch][ldy].
 * 1 <= batch <= QBLK_GEMV_MAX_BATCH.
 * Errors: as qblk_gemv, plus QBLK_ERR_SHAPE for ldx < k and QBLK_ERR_ALIGN
 * for x or ldx.
 */
qblk_status qblk_gemv_float(int type, const void *wq, int64_t n, int64_t k, const float *x,
                    int64_t ldx, int64_t batch, float *y, int64_t ldy,
                    hipStream_t stream);

/*
 * Prefill-path product: the same result as qblk_gemv for m activation rows,
 * Y[m][ldy] = X * W^T, computed with int8 matrix-core tiles. Any m >= 0.
 * Per block the same integer dot and outside scales as qblk_gemv
 * ("llama.cpp 推理引擎", §6.4; wmrh.cn "bare engine" article, §2.2); prefill
 * processes many tokens at once and is compute-bound ("llama.cpp 推理引擎",
 * §7.3), hence the matrix cores. With at most 8 rows the call runs
 * qblk_gemv's kernels where they are faster (m <= 4, n <= 8192, or Q4_K
 * with k a multiple of 2048): results are then qblk_gemv's, bit for bit.
 * Errors as qblk_gemv (no batch limit), plus QBLK_ERR_UNSUPPORTED for
 * k > 2^24.
 */
qblk_status qblk_gemm(int type, const void *wq, int64_t n, int64_t k, const void *xq,
              int64_t m, float *y, int64_t ldy, hipStream_t stream);

/*
 * Quantized KV cache ("llama.cpp 推理引擎", §3.7.1: the cache keeps K and V of
 * every earlier token so that a decode step computes only the new token's;
 * §3.7.3: the cache may be stored as Q8_0 or Q4_0). Types QBLK_Q4_0,
 * QBLK_Q8_0 and QBLK_Q4_0_F16; head_dim 64, 128 or 256.
 *
 * Layout: n_kv heads x n_ctx token rows; row (h, t) is the packed weight row
 * (same layout and encoding as qblk_pack_weights) of the head_dim values of
 * head h at token t, at byte (h * n_ctx + t) * qblk_weight_row_bytes(type,
 * head_dim). The cache is owned by the caller; qblk_kv_cache_bytes gives its
 * size (0 for an invalid type, head_dim, n_kv or n_ctx, or n_kv > 65535).
 */
size_t qblk_kv_cache_bytes(int type, int64_t n_kv, int64_t n_ctx, int64_t head_dim);

/*
 * Store one token: quantize x[h*ldx + i] (h < n_kv, i < head_dim; fp32,
 * 16-byte aligned, ldx a multiple of 4) into rows (h, pos) of the cache, with
 * the qblk_pack_weights rules. The same call serves a K cache and a V cache.
 * Errors: QBLK_ERR_ARG (type, n_kv < 0, null pointers), QBLK_ERR_SHAPE
 * (head_dim, n_ctx <= 0, pos outside [0, n_ctx), ldx < head_dim),
 * QBLK_ERR_ALIGN, QBLK_ERR_UNSUPPORTED (n_kv > 65535), QBLK_ERR_LAUNCH.
 */
qblk_status qblk_kv_store(int type, const float *x, int64_t n_kv, int64_t head_dim, int64_t ldx,
                  void *cache, int64_t n_ctx, int64_t pos, hipStream_t stream);

/*
 * Attention scores against a quantized K cache, the quantized QK^T of a
 * decode step: for query head hq < n_head and token t < n_tok,
 *   scores[hq*lds + t] = sum over 32-blocks j of dk[h][t][j] * dq[hq][j] * S
 * with h = hq / (n_head / n_kv) (grouped queries share a KV head), dk the
 * key block scale, dq the query block scale and S the integer dot of the key
 * codes (Q4_0 / Q4_0_F16: nibble - 8) with the query codes. q is an
 * activation buffer of n_head rows of head_dim (qblk_quantize_act).
 * Accumulation is fp32. No scaling by 1/sqrt(head_dim) and no softmax.
 * Errors: QBLK_ERR_ARG (type, n_kv or n_head <= 0, n_head % n_kv != 0, null
 * pointers), QBLK_ERR_SHAPE (head_dim, n_ctx <= 0, n_tok outside [0, n_ctx],
 * lds < n_tok), QBLK_ERR_ALIGN (cache, q: 16 bytes; scores: 4),
 * QBLK_ERR_UNSUPPORTED (n_head / n_kv > 8, n_kv > 65535), QBLK_ERR_LAUNCH.
 */
qblk_status qblk_kv_scores(int type, const void *cache, int64_t n_kv, int64_t n_ctx, int64_t n_tok,
                   int64_t head_dim, const void *q, int64_t n_head, float *scores, int64_t lds,
                   hipStream_t stream);

/*
 * Test export: the integer block sums S[mm][nn][j] (int32, layout
 * [m][n][k/32]) that qblk_gemv / qblk_gemm scale and accumulate, computed
 * with the same device unpack and dot code: the integer part of the pages'
 * block dot, before any scale ("llama.cpp 推理引擎", §6.4: nibble - 8 times
 * the activation; wmrh.cn "bare engine" article, §2.2: int4 x int8
 * multiply-adds summed to int32). Intended for small shapes.
 * Errors as qblk_gemv (no batch limit).
 */
qblk_status qblk_block_sums(int type, const void *wq, int64_t n, int64_t k,
                    const void *xq, int64_t m, int32_t *sums,
                    hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* QBLK_H */
