// Quantized KV cache: attention scores of the decode step against a K cache
// held in the same 32-block formats as the weights ("llama.cpp 推理引擎",
// §3.7.1: the cache keeps every earlier token's K and V; §3.7.3: the cache
// can be stored as Q8_0 or Q4_0).
//
// Layout: n_kv heads x n_ctx token rows; row (h, t) holds K of token t for KV
// head h as one packed row of head_dim elements (the weight row layout of
// the type) at byte (h * n_ctx + t) * row_bytes. New tokens are written by
// the weight packer with an output row stride of n_ctx rows.
//
// Scores: for query head hq of KV head h = hq / G (G = n_head / n_kv query
// heads share one KV head),
//   scores[hq][t] = sum over 32-blocks j of dk[h][t][j] * dq[hq][j] * S,
// S the integer dot of the key codes with the query's Q8 codes (Q4_0: nibble
// - 8, via the query block sum), as in the weight product.
//
// Mapping: NBH = head_dim / 32 lanes per token, lane j of a token owning
// block j, so a wave step covers 64 / NBH tokens and its loads are whole rows
// of consecutive tokens, all issued before any arithmetic. The query rows of
// one KV head's group are contiguous in the activation buffer: the workgroup
// copies them into LDS once, loading them ahead of the keys so that the copy
// waits for them alone. The per-token sum over the NBH lanes is a butterfly
// of DPP lane moves; the scores pass through an LDS tile so that each query
// head's run of consecutive tokens is written with every lane active.
#include "qblk_device.h"

namespace qblk {
namespace {

constexpr int kMaxGroup = 8;  // query heads per KV head

template <int TYPE, int NBH, int ITER>
__global__ __launch_bounds__(256) void kv_scores_kernel(const uint8_t* __restrict__ cache, int64_t rb,
                                                        int64_t hb, int64_t n_ctx, int64_t n_tok, ActView Q,
                                                        int group, float* __restrict__ scores, int64_t lds) {
  constexpr int kTpw = 64 / NBH;  // tokens per wave and step
  constexpr int kHd = 32 * NBH;   // head_dim
  // one slot per thread, so that every thread stores unconditionally
  __shared__ uint4 qcodes[256];
  __shared__ float2 qds[256];
  static_assert(kMaxGroup * kHd / 16 <= 256 && kMaxGroup * NBH <= 256, "query staging");
  // the workgroup's scores, [query head of the group][token]
  constexpr int kTw = 4 * kTpw * ITER;
  __shared__ float tile[kMaxGroup * kTw];
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int64_t h = blockIdx.y;
  const int j = lane % NBH;
  // this wave's tokens: ITER steps of kTpw consecutive tokens
  const int64_t t0 = (static_cast<int64_t>(blockIdx.x) * 4 + wave) * (kTpw * ITER) + lane / NBH;

  // the group's query rows h * group .. h * group + group - 1 are contiguous
  // in the activation buffer: one copy into LDS per workgroup, loaded before
  // the keys so that the LDS writes wait for these loads only
  const int64_t row0 = h * group;
  const int nqc = group * kHd / 16, nqd = group * NBH;
  const int tid = threadIdx.x;
  const uint4 qv = load16(Q.codes(row0, 0) + 16 * (tid < nqc ? tid : nqc - 1));
  const float2 qdv = Q.dsum(row0, tid < nqd ? tid : nqd - 1);

  // block j of this lane's key rows, all steps issued up front (a padded
  // token re-reads the last one)
  uint4 k0[ITER], k1[ITER];
  float dk[ITER];
#pragma unroll
  for (int it = 0; it < ITER; ++it) {
    const int64_t t = t0 + it * kTpw;
    const int64_t tt = t < n_tok ? t : n_tok - 1;
    const uint8_t* krow = cache + (h * n_ctx + tt) * rb;
    k1[it] = make_uint4(0, 0, 0, 0);
    if constexpr (TYPE == kQ8_0) {
      k0[it] = load_stream16(krow + hb + 32 * j);
      k1[it] = load_stream16(krow + hb + 32 * j + 16);
      dk[it] = __uint_as_float(load_stream4(krow + 4 * j));
    } else {
      k0[it] = load_stream16(krow + hb + 16 * j);
      dk[it] = TYPE == kQ4_0H ? half_bits_to_float(load_stream2(krow + 2 * j))
                              : __uint_as_float(load_stream4(krow + 4 * j));
    }
  }

  qcodes[tid] = qv;
  qds[tid] = qdv;
  __syncthreads();

#pragma unroll
  for (int g = 0; g < kMaxGroup; ++g) {
    if (g < group) {  // uniform
      const uint4 qa0 = qcodes[(g * kHd + 32 * j) / 16], qa1 = qcodes[(g * kHd + 32 * j) / 16 + 1];
      const float2 ds = qds[g * NBH + j];
#pragma unroll
      for (int it = 0; it < ITER; ++it) {
        int s;
        if constexpr (TYPE == kQ8_0)
          s = dot_i8x32(k0[it], k1[it], qa0, qa1, 0);
        else
          s = dot_nib32(k0[it], qa0, qa1, 0) - 8 * __float_as_int(ds.y);  // codes are nibble - 8
        float v = static_cast<float>(s) * dk[it] * ds.x;
        // sum over the token's NBH lanes (aligned groups of 2, 4 or 8)
        v += quad_swap<kQuadXor1>(v);
        if constexpr (NBH >= 4) v += quad_swap<kQuadXor2>(v);
        if constexpr (NBH == 8) v += dpp_move<0x141, 0xF>(v);  // row_half_mirror
        if (j == 0) tile[g * kTw + wave * (kTpw * ITER) + it * kTpw + lane / NBH] = v;
      }
    }
  }
  __syncthreads();
  // rows of kTw consecutive scores, written with every lane active
  const int64_t tok0 = static_cast<int64_t>(blockIdx.x) * kTw;
  for (int e = tid; e < group * kTw; e += 256) {
    const int g = e / kTw, i = e % kTw;
    const int64_t t = tok0 + i;
    if (t < n_tok) scores[(row0 + g) * lds + t] = tile[e];
  }
}

// Token steps per wave. One step in 4 x more workgroups beats two or four
// steps per wave (Q8_0, 8 KV heads of 128, 64 query heads, 32768 tokens:
// 13.3 us at one step, 15.3 us at two).
constexpr int kIter = 1;

template <int TYPE, int NBH>
void launch_nbh(const uint8_t* cache, int64_t rb, int64_t hb, int64_t n_kv, int64_t n_ctx, int64_t n_tok,
                const ActView& Q, int group, float* scores, int64_t lds, hipStream_t s) {
  constexpr int64_t kTokensPerWg = 4 * (64 / NBH) * kIter;
  const dim3 grid(static_cast<uint32_t>((n_tok + kTokensPerWg - 1) / kTokensPerWg), static_cast<uint32_t>(n_kv));
  hipLaunchKernelGGL((kv_scores_kernel<TYPE, NBH, kIter>), grid, dim3(256), 0, s, cache, rb, hb, n_ctx, n_tok, Q,
                     group, scores, lds);
}

template <int TYPE>
void launch_type(const uint8_t* cache, int64_t rb, int64_t hb, int64_t n_kv, int64_t n_ctx, int64_t n_tok,
                 int64_t head_dim, const ActView& Q, int group, float* scores, int64_t lds, hipStream_t s) {
  switch (head_dim) {
    case 64: launch_nbh<TYPE, 2>(cache, rb, hb, n_kv, n_ctx, n_tok, Q, group, scores, lds, s); break;
    case 128: launch_nbh<TYPE, 4>(cache, rb, hb, n_kv, n_ctx, n_tok, Q, group, scores, lds, s); break;
    default: launch_nbh<TYPE, 8>(cache, rb, hb, n_kv, n_ctx, n_tok, Q, group, scores, lds, s); break;
  }
}

}  // namespace

hipError_t launch_kv_scores(int type, const void* cache, int64_t n_kv, int64_t n_ctx, int64_t n_tok,
                            int64_t head_dim, const void* q, int64_t n_head, float* scores, int64_t lds,
                            hipStream_t s) {
  const auto* c = static_cast<const uint8_t*>(cache);
  const int64_t rb = row_bytes(type, head_dim);
  const int64_t hb = header_bytes(type, head_dim);
  const ActView Q = make_act(q, n_head, head_dim);
  const int group = static_cast<int>(n_head / n_kv);
  switch (type) {
    case kQ8_0: launch_type<kQ8_0>(c, rb, hb, n_kv, n_ctx, n_tok, head_dim, Q, group, scores, lds, s); break;
    case kQ4_0H: launch_type<kQ4_0H>(c, rb, hb, n_kv, n_ctx, n_tok, head_dim, Q, group, scores, lds, s); break;
    default: launch_type<kQ4_0>(c, rb, hb, n_kv, n_ctx, n_tok, head_dim, Q, group, scores, lds, s); break;
  }
  return hipGetLastError();
}

}  // namespace qblk
