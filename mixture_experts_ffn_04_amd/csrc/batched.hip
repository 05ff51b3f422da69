// The "batched_mm" expert execution (article "Mixture of Experts (MoEs) in
// Transformers", section "Expert Backend"): for small batches, every
// routed (token, slot) pair is multiplied with the weights of the expert it
// selected, as one batched product over the pairs, with no sort by expert.
// The article's form copies the selected weights per token before a batched
// GEMM; here each pair reads them in place through its expert id, so
// nothing is copied.  The down projection folds in the weighted sum over a
// token's k slots, in increasing slot order and without atomics, so no
// combine pass or permutation is needed.
//
// An expert chosen by several pairs is read once per pair, so the strategy
// suits batches whose pairs seldom share an expert (one decoding token never
// does: its k experts are distinct).  Each wave streams two weight rows in
// 16-byte loads (1 KB per load instruction, a plain streaming read) and
// reduces their dot products with the pair's activation row across the wave.
#include "common.h"
#include "select.h"

namespace moe {
namespace {

typedef __attribute__((address_space(1))) const u32x4 gu4;

constexpr int64_t kBatchedMaxPairs = 1024;
constexpr int kSegChunks = 8;   // 16-byte chunks per lane per K segment (4096 bf16 elements)

// Per-lane partial dot products of weight rows w0, w1 with activation row x
// (KC 16-byte chunks each): lane l takes chunks l, l + 64, ...; each
// segment's loads are all issued before its arithmetic.
__device__ __forceinline__ void dot_rows2(const gu4* w0, const gu4* w1, const gu4* x, int KC, int lane, float& a,
                                          float& b) {
  const u32x4 zero = {0u, 0u, 0u, 0u};
  for (int base = 0; base < KC; base += 64 * kSegChunks) {
    u32x4 v0[kSegChunks], v1[kSegChunks], xv[kSegChunks];
#pragma unroll
    for (int i = 0; i < kSegChunks; ++i) {
      const int c = base + lane + 64 * i;
      const bool ok = c < KC;
      v0[i] = ok ? w0[c] : zero;
      v1[i] = ok ? w1[c] : zero;
      xv[i] = ok ? x[c] : zero;
    }
#pragma unroll
    for (int i = 0; i < kSegChunks; ++i) {
      a = dot8(v0[i], xv[i], a);
      b = dot8(v1[i], xv[i], b);
    }
  }
}

__device__ __forceinline__ void wave_sum2(float& a, float& b) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) {
    a += __shfl_xor(a, o, 64);
    b += __shfl_xor(b, o, 64);
  }
}

// h[p][n] = silu(x[p/k] . Wg[e][n]) * (x[p/k] . Wu[e][n]), e = ids[p].
// Workgroup = (pair p, 4 output columns), one column (its gate and up
// rows) per wave.  Pairs with an id outside [0, E) get no row.
// S > 0: the experts are selected here from the router logits [T][E] (every
// wave runs its token's selection, S candidate slots per lane), and the
// first workgroup of each token writes the token's ids and weights.
template <int S>
__global__ __launch_bounds__(256) void batched_gateup_kernel(const u32x4* __restrict__ x,
                                                             int32_t* __restrict__ ids, const float* __restrict__ logits,
                                                             int score, float* __restrict__ wts,
                                                             const u32x4* __restrict__ W, int P, int k, int E,
                                                             int K, int N, uint16_t* __restrict__ h) {
  const int ncb = N / 4;
  const int p = blockIdx.x / ncb;
  const int cb = blockIdx.x - p * ncb;
  const int n = cb * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (p >= P) return;
  int e;
  if constexpr (S > 0) {
    const int t = p / k, j = p - t * k;
    float sel_v[kMaxK];
    int sel_i[kMaxK];
    topk_select<S>(logits + static_cast<int64_t>(t) * E, E, k, sel_v, sel_i);
    if (j == 0 && cb == 0 && threadIdx.x == 0)
      topk_store(sel_v, sel_i, k, score, ids + static_cast<int64_t>(t) * k, wts + static_cast<int64_t>(t) * k);
    e = topk_slot(sel_i, k, j);
  } else {
    e = ids[p];
  }
  if (e < 0 || e >= E) return;                       // a pair of an expert held elsewhere
  const int KC = K / 8;
  const gu4* We = (const gu4*)W + static_cast<int64_t>(e) * 2 * N * KC;
  float a = 0.0f, b = 0.0f;
  dot_rows2(We + static_cast<int64_t>(n) * KC, We + static_cast<int64_t>(N + n) * KC,
            (const gu4*)x + static_cast<int64_t>(p / k) * KC, KC, lane, a, b);
  wave_sum2(a, b);
  if (lane == 0) h[static_cast<int64_t>(p) * N + n] = f32_to_bf16(silu(a) * b);
}

// y[t][c] = sum_j w[t][j] * (h[t*k+j] . Wd[e_tj][c])  (+ y_shared[t][c]),
// the sum in fp32 in increasing j, then the shared row, rounded once.
// Workgroup = (token t, 2 output columns); wave w takes slots j = w, w+4,
// ..., each slot's two dot products go to LDS, and one thread per column
// sums them in slot order.  Slots with an id outside [0, E) add nothing.
__global__ __launch_bounds__(256) void batched_down_combine_kernel(const u32x4* __restrict__ h,
                                                                   const int32_t* __restrict__ ids,
                                                                   const float* __restrict__ wts,
                                                                   const u32x4* __restrict__ W,
                                                                   const uint16_t* __restrict__ ys, int T, int k,
                                                                   int E, int K, int N, uint16_t* __restrict__ y) {
  __shared__ float part[kMaxK][2];
  const int ncb = N / 2;
  const int t = blockIdx.x / ncb;
  const int c0 = (blockIdx.x - t * ncb) * 2;
  if (t >= T) return;                                // uniform over the workgroup
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int KC = K / 8;
  for (int j = wave; j < k; j += 4) {
    const int64_t p = static_cast<int64_t>(t) * k + j;
    const int e = ids[p];
    float a = 0.0f, b = 0.0f;
    if (e >= 0 && e < E) {
      const gu4* We = (const gu4*)W + static_cast<int64_t>(e) * N * KC;
      dot_rows2(We + static_cast<int64_t>(c0) * KC, We + static_cast<int64_t>(c0 + 1) * KC,
                (const gu4*)h + p * KC, KC, lane, a, b);
      wave_sum2(a, b);
    }
    if (lane == 0) {
      part[j][0] = a;
      part[j][1] = b;
    }
  }
  __syncthreads();
  if (threadIdx.x < 2) {
    const int c = c0 + threadIdx.x;
    float acc = 0.0f;
    for (int j = 0; j < k; ++j) {
      const int64_t p = static_cast<int64_t>(t) * k + j;
      const int e = ids[p];
      if (e >= 0 && e < E) acc = fmaf(wts[p], part[j][threadIdx.x], acc);
    }
    const int64_t o = static_cast<int64_t>(t) * N + c;
    if (ys) acc += bf16_to_f32(ys[o]);
    y[o] = f32_to_bf16(acc);
  }
}

moe_status check_batched(const void* in, const int32_t* ids, const void* w, int64_t T, int64_t d, int64_t f,
                         int32_t E, int32_t k, moe_dtype dtype, const void* out) {
  if (T < 0 || d <= 0 || f <= 0 || E < 1 || k < 1 || k > kMaxK || !valid_dtype(dtype)) return MOE_ERR_INVALID_ARG;
  if (E > kMaxE || dtype != MOE_BF16) return MOE_ERR_UNSUPPORTED;
  if (d % 64 != 0 || f % 64 != 0) return MOE_ERR_ALIGNMENT;
  if (T * k > kBatchedMaxPairs) return MOE_ERR_UNSUPPORTED;
  if (T == 0) return MOE_OK;
  if (!in || !ids || !w || !out) return MOE_ERR_INVALID_ARG;
  if (!aligned16(in) || !aligned16(w)) return MOE_ERR_ALIGNMENT;
  return MOE_OK;
}

}  // namespace
}  // namespace moe

using namespace moe;

extern "C" moe_status moe_batched_gateup_swiglu(const void* x, const int32_t* topk_ids, const void* w_gate_up,
                                                int64_t T, int64_t d, int64_t f, int32_t E, int32_t k,
                                                moe_dtype dtype, void* h, void* stream) {
  moe_status s = check_batched(x, topk_ids, w_gate_up, T, d, f, E, k, dtype, h);
  if (s != MOE_OK || T == 0) return s;
  const int64_t P = T * k;
  hipLaunchKernelGGL(batched_gateup_kernel<0>, dim3(static_cast<unsigned>(P * (f / 4))), dim3(256), 0,
                     as_stream(stream), static_cast<const u32x4*>(x), const_cast<int32_t*>(topk_ids), nullptr, 0,
                     nullptr, static_cast<const u32x4*>(w_gate_up), static_cast<int>(P), k, E, static_cast<int>(d),
                     static_cast<int>(f), static_cast<uint16_t*>(h));
  return launch_status();
}

extern "C" moe_status moe_batched_gateup_swiglu_select(const void* x, const float* logits, const void* w_gate_up,
                                                       int64_t T, int64_t d, int64_t f, int32_t E, int32_t k,
                                                       moe_score score, moe_dtype dtype, int32_t* topk_ids,
                                                       float* topk_w, void* h, void* stream) {
  moe_status s = check_batched(x, logits ? topk_ids : nullptr, w_gate_up, T, d, f, E, k, dtype, h);
  if (s != MOE_OK || T == 0) return s;
  if (!topk_w || k > E || (score != MOE_SCORE_SOFTMAX && score != MOE_SCORE_SIGMOID)) return MOE_ERR_INVALID_ARG;
  const int64_t P = T * k;
#define MOE_BGU_SEL(S_)                                                                                          \
  hipLaunchKernelGGL(batched_gateup_kernel<S_>, dim3(static_cast<unsigned>(P * (f / 4))), dim3(256), 0,            \
                     as_stream(stream), static_cast<const u32x4*>(x), topk_ids, logits, static_cast<int>(score),    \
                     topk_w, static_cast<const u32x4*>(w_gate_up), static_cast<int>(P), k, E, static_cast<int>(d),   \
                     static_cast<int>(f), static_cast<uint16_t*>(h))
  if (E <= 64)
    MOE_BGU_SEL(1);
  else if (E <= 128)
    MOE_BGU_SEL(2);
  else
    MOE_BGU_SEL(4);
#undef MOE_BGU_SEL
  return launch_status();
}

extern "C" moe_status moe_batched_down_combine(const void* h, const int32_t* topk_ids, const float* topk_w,
                                               const void* w_down, const void* y_shared, int64_t T, int64_t d,
                                               int64_t f, int32_t E, int32_t k, moe_dtype dtype, void* y,
                                               void* stream) {
  moe_status s = check_batched(h, topk_ids, w_down, T, d, f, E, k, dtype, y);
  if (s != MOE_OK || T == 0) return s;
  if (!topk_w) return MOE_ERR_INVALID_ARG;
  hipLaunchKernelGGL(batched_down_combine_kernel, dim3(static_cast<unsigned>(T * (d / 2))), dim3(256), 0,
                     as_stream(stream), static_cast<const u32x4*>(h), topk_ids, topk_w,
                     static_cast<const u32x4*>(w_down), static_cast<const uint16_t*>(y_shared),
                     static_cast<int>(T), k, E, static_cast<int>(f), static_cast<int>(d), static_cast<uint16_t*>(y));
  return launch_status();
}
