// Router: logits, top-k selection and routing weights.
//
// Article "Mixture of Experts (MoEs) in Transformers", section "From Dense
// to Sparse": per token, a few experts are chosen from scores computed on
// the token's activations.
//
// Logits are a dense contraction x[T][d] . w_router[E][d]^T, computed by the
// grouped GEMM kernels as a single group with a "+ bias, fp32" epilogue, or
// for small batches by the split-K streaming kernel of the decode path.
//
// Selection and weights: one wave per token (select.h), with 1, 2 or 4
// candidate slots per lane for E <= 64, 128, 256.
#include "grouped_gemm.h"
#include "select.h"

namespace moe {

moe_status gemm_bf16_logits(const GemmArgs& a, hipStream_t st);
moe_status gemm_f32_logits(const GemmArgs& a, hipStream_t st);
moe_status decode_bf16_logits(const void* x, const void* w_router, const float* bias, int64_t T, int64_t d,
                              int32_t E, float* logits, hipStream_t st, int rb);

// bf16 router logits, by size (measured on MI355X):
//  - T*E <= kTinyRouteItems (d <= 8192): one wave per (expert row, few
//    tokens), every load issued up front;
//  - E <= kStreamRouteExperts or T <= kStreamRouteTokens: the streaming
//    split-K kernel with the tokens split into blocks of 16 (32 once
//    16-token blocks would make at least kStreamRouteBlocks workgroups),
//    one workgroup per (16 experts, token block);
//  - above: the tiled MFMA GEMM, which reuses tokens across 128 experts.
constexpr int64_t kTinyRouteItems = 8192;
constexpr int kStreamRouteExperts = 64;
constexpr int64_t kStreamRouteTokens = 1024;
constexpr int64_t kStreamRouteBlocks = 1024;

namespace {

constexpr int kTokPerBlock = 4;   // one wave each

template <int S>
__global__ __launch_bounds__(256) void topk_kernel(const float* __restrict__ logits, int T, int E, int k,
                                                   int score, int32_t* __restrict__ ids,
                                                   float* __restrict__ wts) {
  const int tok = blockIdx.x * kTokPerBlock + (threadIdx.x >> 6);
  if (tok >= T) return;
  float sel_v[kMaxK];
  int sel_i[kMaxK];
  topk_select<S>(logits + static_cast<int64_t>(tok) * E, E, k, sel_v, sel_i);
  if ((threadIdx.x & 63) == 0)
    topk_store(sel_v, sel_i, k, score, ids + static_cast<int64_t>(tok) * k, wts + static_cast<int64_t>(tok) * k);
}

// Small batches (bf16): router logits with one wave per (expert, block of
// TOK tokens).  Every load of the wave -- its NCH 16-byte chunks of the
// expert's row and of each token's row -- is issued before any arithmetic,
// so the whole router matrix and the tokens are requested in one round
// trip.  Each logit is an fp32 dot product of 8-element chunks summed
// across the wave, plus the bias.  d <= 64 * 8 * NCH.
template <int NCH, int TOK>
__global__ __launch_bounds__(256) void logits_small_kernel(const uint16_t* __restrict__ x,
                                                           const uint16_t* __restrict__ wr,
                                                           const float* __restrict__ bias, int T, int d, int E,
                                                           float* __restrict__ logits) {
  const int lane = threadIdx.x & 63;
  const int item = blockIdx.x * 4 + (threadIdx.x >> 6);       // (token block, expert), expert fastest
  const int e = item % E;
  const int t0 = (item / E) * TOK;
  if (t0 >= T) return;
  const int nt = min(TOK, T - t0);
  const int nc = d / 8;
  const uint16_t* w = wr + static_cast<int64_t>(e) * d;
  const u32x4 zero = {0u, 0u, 0u, 0u};
  u32x4 wv[NCH];
  u32x4 xv[TOK][NCH];
#pragma unroll
  for (int j = 0; j < NCH; ++j) {
    const int c = lane + 64 * j;
    wv[j] = c < nc ? *reinterpret_cast<const u32x4*>(w + c * 8) : zero;
  }
#pragma unroll
  for (int i = 0; i < TOK; ++i) {
    const uint16_t* xt = x + static_cast<int64_t>(t0 + (i < nt ? i : 0)) * d;
#pragma unroll
    for (int j = 0; j < NCH; ++j) {
      const int c = lane + 64 * j;
      xv[i][j] = c < nc ? *reinterpret_cast<const u32x4*>(xt + c * 8) : zero;
    }
  }
  float acc[TOK];
#pragma unroll
  for (int i = 0; i < TOK; ++i) {
    acc[i] = 0.0f;
#pragma unroll
    for (int j = 0; j < NCH; ++j) {
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        acc[i] += bf16_to_f32(static_cast<uint16_t>(wv[j][q] & 0xffffu)) *
                  bf16_to_f32(static_cast<uint16_t>(xv[i][j][q] & 0xffffu));
        acc[i] += bf16_to_f32(static_cast<uint16_t>(wv[j][q] >> 16)) * bf16_to_f32(static_cast<uint16_t>(xv[i][j][q] >> 16));
      }
    }
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) acc[i] += __shfl_xor(acc[i], o, 64);
  }
  if (lane == 0) {
    const float b = bias ? bias[e] : 0.0f;
#pragma unroll
    for (int i = 0; i < TOK; ++i)
      if (i < nt) logits[static_cast<int64_t>(t0 + i) * E + e] = acc[i] + b;
  }
}

template <int NCH, int TOK>
moe_status launch_logits_small(const void* x, const void* w_router, const float* bias, int64_t T, int64_t d,
                               int32_t E, float* logits, hipStream_t st) {
  const int64_t items = ceil_div(T, TOK) * E;
  hipLaunchKernelGGL((logits_small_kernel<NCH, TOK>), dim3(static_cast<unsigned>(ceil_div(items, 4))), dim3(256), 0,
                     st, static_cast<const uint16_t*>(x), static_cast<const uint16_t*>(w_router), bias,
                     static_cast<int>(T), static_cast<int>(d), E, logits);
  return launch_status();
}

moe_status check_topk_args(int64_t T, int32_t E, int32_t k, moe_score score) {
  if (T < 0 || E < 1 || k < 1 || k > E || k > kMaxK) return MOE_ERR_INVALID_ARG;
  if (E > kMaxE) return MOE_ERR_UNSUPPORTED;
  if (T * static_cast<int64_t>(k) >= (int64_t(1) << 31)) return MOE_ERR_UNSUPPORTED;
  if (score != MOE_SCORE_SOFTMAX && score != MOE_SCORE_SIGMOID) return MOE_ERR_INVALID_ARG;
  return MOE_OK;
}

moe_status launch_topk(const float* logits, int64_t T, int32_t E, int32_t k, moe_score score,
                       int32_t* ids, float* w, hipStream_t st) {
  const int64_t blocks = ceil_div(T, kTokPerBlock);
  // candidate slots per lane: 1 (E <= 64), 2 (E <= 128) or 4
#define MOE_TOPK(S_)                                                                                  \
  hipLaunchKernelGGL(topk_kernel<S_>, dim3(static_cast<unsigned>(blocks)), dim3(256), 0, st, logits, \
                     static_cast<int>(T), E, k, static_cast<int>(score), ids, w)
  if (E <= 64)
    MOE_TOPK(1);
  else if (E <= 128)
    MOE_TOPK(2);
  else
    MOE_TOPK(4);
#undef MOE_TOPK
  return launch_status();
}

}  // namespace
}  // namespace moe

using namespace moe;

extern "C" moe_status moe_topk(const float* logits, int64_t T, int32_t E, int32_t k, moe_score score,
                               int32_t* topk_ids, float* topk_w, void* stream) {
  moe_status s = check_topk_args(T, E, k, score);
  if (s != MOE_OK) return s;
  if (T == 0) return MOE_OK;
  if (!logits || !topk_ids || !topk_w) return MOE_ERR_INVALID_ARG;
  return launch_topk(logits, T, E, k, score, topk_ids, topk_w, as_stream(stream));
}

extern "C" moe_status moe_route(const void* x, const void* w_router, const float* bias, int64_t T,
                                int64_t d, int32_t E, int32_t k, moe_dtype dtype, moe_score score,
                                float* logits, int32_t* topk_ids, float* topk_w, void* stream) {
  moe_status s = check_topk_args(T, E, k, score);
  if (s != MOE_OK) return s;
  if (!valid_dtype(dtype) || d <= 0) return MOE_ERR_INVALID_ARG;
  if (d % 64 != 0) return MOE_ERR_ALIGNMENT;
  if (T == 0) return MOE_OK;
  if (!x || !w_router || !logits || (!topk_ids) != (!topk_w)) return MOE_ERR_INVALID_ARG;
  if (!aligned16(x) || !aligned16(w_router) || !aligned16(logits)) return MOE_ERR_ALIGNMENT;
  GemmArgs a{};
  a.A = x;
  a.B = w_router;
  a.off = nullptr;
  a.bias = bias;
  a.C = logits;
  a.rows = T;
  a.K = d;
  a.N = E;
  a.G = 1;
  hipStream_t st = as_stream(stream);
  const bool tiny = T * E <= kTinyRouteItems;
  const bool stream_ok = (E <= kStreamRouteExperts || T <= kStreamRouteTokens) && ceil_div(T, 16) <= 65535;
  if (dtype == MOE_BF16 && tiny && d <= 4096) {
    s = launch_logits_small<8, 4>(x, w_router, bias, T, d, E, logits, st);
  } else if (dtype == MOE_BF16 && tiny && d <= 8192) {
    s = launch_logits_small<16, 2>(x, w_router, bias, T, d, E, logits, st);
  } else if (dtype == MOE_BF16 && stream_ok) {
    const int rb = ceil_div(T, 16) * ceil_div(E, 16) < kStreamRouteBlocks ? 16 : 32;
    s = decode_bf16_logits(x, w_router, bias, T, d, E, logits, st, rb);
  } else {
    s = (dtype == MOE_BF16) ? gemm_bf16_logits(a, st) : gemm_f32_logits(a, st);
  }
  if (s != MOE_OK || !topk_ids) return s;                 // logits only
  return launch_topk(logits, T, E, k, score, topk_ids, topk_w, st);
}
