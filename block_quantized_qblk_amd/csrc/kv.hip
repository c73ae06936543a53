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
// Mapping: a token's row is read by L consecutive lanes, each taking 16
// contiguous bytes: for Q4_0 a whole block of nibbles (L = head_dim / 32),
// for Q8_0 half a block (L = head_dim / 16), so that the L lanes read the
// row's codes as one contiguous run (two interleaved 16-B loads per Q8_0
// block are about a third slower). A wave step covers 64 / L consecutive
// tokens; all of a wave's key loads are issued before any arithmetic. The
// query rows of one KV head's group are contiguous in the activation buffer:
// the workgroup copies them into LDS once, loading them ahead of the keys so
// that the copy waits for them alone. A Q8_0 block's two integer half-dots
// are added exactly across the lane pair before the block is scaled; the
// per-token sum over blocks is a butterfly of DPP lane moves. The scores pass
// through an LDS tile so that each query head's run of consecutive tokens is
// written with every lane active.
#include "qblk_device.h"

namespace qblk {
namespace {

constexpr int kMaxGroup = 8;  // query heads per KV head

// Lanes per token row.
template <int TYPE, int NBH>
constexpr int lanes_per_token() {
  return TYPE == kQ8_0 ? 2 * NBH : NBH;
}

template <int TYPE, int NBH, int ITER>
constexpr int tokens_per_workgroup() {
  return 4 * (64 / lanes_per_token<TYPE, NBH>()) * ITER;
}

template <int TYPE, int NBH, int ITER>
__global__ __launch_bounds__(256) void kv_scores_kernel(const uint8_t* __restrict__ cache, int64_t rb,
                                                        int64_t hb, int64_t n_ctx, int64_t n_tok, ActView Q,
                                                        int group, float* __restrict__ scores, int64_t lds) {
  constexpr bool kHalf = TYPE == kQ8_0;  // a lane holds 16 of its block's 32 codes
  constexpr int kL = lanes_per_token<TYPE, NBH>();
  constexpr int kTpw = 64 / kL;  // tokens per wave and step
  constexpr int kIter = ITER;
  constexpr int kHd = 32 * NBH;  // head_dim
  constexpr int kTw = tokens_per_workgroup<TYPE, NBH, ITER>();
  // one slot per thread, so that every thread stores unconditionally
  __shared__ uint4 qcodes[256];
  __shared__ float2 qds[256];
  static_assert(kMaxGroup * kHd / 16 <= 256 && kMaxGroup * NBH <= 256, "query staging");
  // the workgroup's scores, [query head of the group][token]
  __shared__ float tile[kMaxGroup * kTw];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int64_t h = blockIdx.y;
  const int p = lane % kL;          // 16-B piece of the row's codes
  const int j = kHalf ? p >> 1 : p;  // its block
  // this wave's tokens: kIter steps of kTpw consecutive tokens
  const int64_t t0 = (static_cast<int64_t>(blockIdx.x) * 4 + wave) * (kTpw * kIter) + lane / kL;

  // the group's query rows h * group .. h * group + group - 1, loaded before
  // the keys so that the LDS writes wait for these loads only
  const int64_t row0 = h * group;
  const int nqc = group * kHd / 16, nqd = group * NBH;
  const uint4 qv = load16(Q.codes(row0, 0) + 16 * (tid < nqc ? tid : nqc - 1));
  const float2 qdv = Q.dsum(row0, tid < nqd ? tid : nqd - 1);

  // piece p of this lane's key rows, all steps issued up front (a padded
  // token re-reads the last one)
  uint4 kc[kIter];
  float dk[kIter];
#pragma unroll
  for (int it = 0; it < kIter; ++it) {
    const int64_t t = t0 + it * kTpw;
    const int64_t tt = t < n_tok ? t : n_tok - 1;
    const uint8_t* krow = cache + (h * n_ctx + tt) * rb;
    kc[it] = load_stream16(krow + hb + 16 * p);
    dk[it] = TYPE == kQ4_0H ? half_bits_to_float(load_stream2(krow + 2 * j))
                            : __uint_as_float(load_stream4(krow + 4 * j));
  }

  qcodes[tid] = qv;
  qds[tid] = qdv;
  __syncthreads();

#pragma unroll
  for (int g = 0; g < kMaxGroup; ++g) {
    if (g < group) {  // uniform
      const float2 ds = qds[g * NBH + j];
      uint4 qa0, qa1;
      if constexpr (kHalf) {
        qa0 = qcodes[g * kHd / 16 + p];
      } else {
        qa0 = qcodes[g * kHd / 16 + 2 * j];
        qa1 = qcodes[g * kHd / 16 + 2 * j + 1];
      }
#pragma unroll
      for (int it = 0; it < kIter; ++it) {
        int s;
        if constexpr (kHalf) {
          s = dot4_zero(kc[it].x, qa0.x);
          s = dot4(kc[it].y, qa0.y, s);
          s = dot4(kc[it].z, qa0.z, s);
          s = dot4(kc[it].w, qa0.w, s);
          s += quad_swap<kQuadXor1>(s);  // the block's other half (exact)
        } else {
          s = dot_nib32(kc[it], qa0, qa1) - 8 * __float_as_int(ds.y);  // codes are nibble - 8
        }
        float v = static_cast<float>(s) * dk[it] * ds.x;
        // sum over the token's blocks: lanes hold one block each (Q4_0) or
        // one block per lane pair (Q8_0), in aligned groups of 2 to 16 lanes
        if constexpr (!kHalf) v += quad_swap<kQuadXor1>(v);
        if constexpr (kL >= 4) v += quad_swap<kQuadXor2>(v);
        if constexpr (kL >= 8) v += dpp_move<0x141, 0xF>(v);  // row_half_mirror
        if constexpr (kL >= 16) v += dpp_move<0x140, 0xF>(v);  // row_mirror
        if (p == 0) tile[g * kTw + wave * (kTpw * kIter) + it * kTpw + lane / kL] = v;
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

template <int TYPE, int NBH, int ITER>
void launch_iter(const uint8_t* cache, int64_t rb, int64_t hb, int64_t n_kv, int64_t n_ctx, int64_t n_tok,
                 const ActView& Q, int group, float* scores, int64_t lds, hipStream_t s) {
  constexpr int64_t kTw = tokens_per_workgroup<TYPE, NBH, ITER>();
  const dim3 grid(static_cast<uint32_t>((n_tok + kTw - 1) / kTw), static_cast<uint32_t>(n_kv));
  hipLaunchKernelGGL((kv_scores_kernel<TYPE, NBH, ITER>), grid, dim3(256), 0, s, cache, rb, hb, n_ctx, n_tok, Q,
                     group, scores, lds);
}

// Token steps per wave: one, or two for Q8_0 over many rows. Measured on
// MI355X (Q8_0, 8 KV heads of 128, 64 query heads): 8192 tokens 5.07 us at one
// step against 5.37 at two; 32768 tokens 13.7 against 12.8 us; four steps
// no better.
template <int TYPE, int NBH>
void launch_nbh(const uint8_t* cache, int64_t rb, int64_t hb, int64_t n_kv, int64_t n_ctx, int64_t n_tok,
                const ActView& Q, int group, float* scores, int64_t lds, hipStream_t s) {
  if (TYPE == kQ8_0 && n_kv * n_tok >= (int64_t{1} << 17))
    launch_iter<TYPE, NBH, 2>(cache, rb, hb, n_kv, n_ctx, n_tok, Q, group, scores, lds, s);
  else
    launch_iter<TYPE, NBH, 1>(cache, rb, hb, n_kv, n_ctx, n_tok, Q, group, scores, lds, s);
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
