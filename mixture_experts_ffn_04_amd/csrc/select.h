// Top-k selection and routing weights of one token, by one wave (article
// "Mixture of Experts (MoEs) in Transformers", section "From Dense to
// Sparse": per token a few experts are chosen from router scores).
//
// Lane l holds logits l, l+64, ... in S slots (E <= 64 S).  Each of the k
// rounds takes the largest key over the wave, then the lowest index holding
// it, and retires that candidate: larger logit first, equal logits to the
// lower index.  The k winners in selection order give the weights: a
// softmax over the selected logits, or sigmoid scores divided by their sum.
// Used by the router's top-k kernel and by the batched_mm gate/up calls
// that select their own experts, so both produce the same ids and weights.
#pragma once

#include "common.h"

namespace moe {

// Order-preserving 32-bit key of a logit: unsigned comparison of keys is
// the float comparison (-0 is taken as +0, so the two tie); 0 lies below
// every real key and marks "no candidate".
__device__ __forceinline__ unsigned logit_key(float f) {
  unsigned u = __float_as_uint(f);
  if (u == 0x80000000u) u = 0u;
  return (u >> 31) ? ~u : (u | 0x80000000u);
}

__device__ __forceinline__ float key_logit(unsigned k) {
  return __uint_as_float((k >> 31) ? (k & 0x7fffffffu) : ~k);
}

// Maximum over the wave, in every lane: an inclusive max-scan inside each
// 16-lane row by DPP row shifts of 1, 2, 4, 8, then the row totals carried
// across rows by row_bcast 15 and 31, so lane 63 holds the wave's maximum.
__device__ __forceinline__ unsigned wave_max(unsigned v) {
  int x = static_cast<int>(v);
#define MOE_MAX_DPP(ctrl, rows)                                                                  \
  x = static_cast<int>(max(static_cast<unsigned>(x),                                            \
                           static_cast<unsigned>(__builtin_amdgcn_update_dpp(0, x, ctrl, rows, 0xf, false))))
  MOE_MAX_DPP(0x111, 0xf);   // row_shr:1
  MOE_MAX_DPP(0x112, 0xf);   // row_shr:2
  MOE_MAX_DPP(0x114, 0xf);   // row_shr:4
  MOE_MAX_DPP(0x118, 0xf);   // row_shr:8
  MOE_MAX_DPP(0x142, 0xa);   // row_bcast:15 into rows 1 and 3
  MOE_MAX_DPP(0x143, 0xc);   // row_bcast:31 into rows 2 and 3
#undef MOE_MAX_DPP
  return static_cast<unsigned>(__builtin_amdgcn_readlane(x, 63));
}

// The k selections of one token (row = its E logits, global memory or LDS),
// wave-uniform: sel_i[j] the expert of slot j, sel_v[j] its logit.
template <int S>
__device__ __forceinline__ void topk_select(const float* row, int E, int k, float (&sel_v)[kMaxK],
                                            int (&sel_i)[kMaxK]) {
  const int lane = threadIdx.x & 63;
  float v[S];
#pragma unroll
  for (int i = 0; i < S; ++i) {                 // every logit requested before any is used
    const int e = lane + 64 * i;
    v[i] = row[e < E ? e : 0];
  }
  unsigned key[S];
#pragma unroll
  for (int i = 0; i < S; ++i) key[i] = lane + 64 * i < E ? logit_key(v[i]) : 0u;
#pragma unroll
  for (int j = 0; j < kMaxK; ++j) {
    if (j >= k) break;
    unsigned lm = key[0];
#pragma unroll
    for (int i = 1; i < S; ++i) lm = max(lm, key[i]);
    const unsigned m = wave_max(lm);
    int e = -1;
#pragma unroll
    for (int i = 0; i < S; ++i) {
      const uint64_t b = __ballot(key[i] == m);
      if (e < 0 && b != 0) e = 64 * i + static_cast<int>(__builtin_ctzll(b));
    }
    sel_v[j] = key_logit(m);
    sel_i[j] = e;
#pragma unroll
    for (int i = 0; i < S; ++i)
      if (lane + 64 * i == e) key[i] = 0u;
  }
}

// The routing weights of the k selections, written with their ids by the
// calling lane (ids[j], wts[j] for j < k).
__device__ __forceinline__ void topk_store(const float (&sel_v)[kMaxK], const int (&sel_i)[kMaxK], int k, int score,
                                           int32_t* __restrict__ ids, float* __restrict__ wts) {
  float w[kMaxK];
  float s = 0.0f;
  if (score == MOE_SCORE_SOFTMAX) {
    const float m = sel_v[0];
#pragma unroll
    for (int j = 0; j < kMaxK; ++j) {
      if (j >= k) break;
      w[j] = expf(sel_v[j] - m);
      s += w[j];
    }
  } else {
#pragma unroll
    for (int j = 0; j < kMaxK; ++j) {
      if (j >= k) break;
      w[j] = 1.0f / (1.0f + expf(-sel_v[j]));
      s += w[j];
    }
  }
  const float inv = 1.0f / s;
#pragma unroll
  for (int j = 0; j < kMaxK; ++j) {
    if (j >= k) break;
    ids[j] = sel_i[j];
    wts[j] = w[j] * inv;
  }
}

// sel_i[j] for a runtime slot j (a chain of selects: no indexed register
// array).
__device__ __forceinline__ int topk_slot(const int (&sel_i)[kMaxK], int k, int j) {
  int e = -1;
#pragma unroll
  for (int jj = 0; jj < kMaxK; ++jj)
    if (jj < k && jj == j) e = sel_i[jj];
  return e;
}

}  // namespace moe
