// Apply the routing weights and collect the expert outputs back in token
// order -- the last step an expert execution strategy performs (article
// "Mixture of Experts (MoEs) in Transformers", section "Expert Backend").
//
//   y[t] = sum_{j<k} w[t][j] * y_perm[inv_perm[t*k + j]]  (+ y_shared[t])
//
// One wave per token row; each lane owns 16-byte column chunks (8 bf16 or
// 4 fp32) and sums its k gathered rows in fp32 in increasing j, then the
// shared-expert row, then rounds once.  Reads and writes are 16-byte and
// coalesced along the row; no atomics, so the result is deterministic.
#include "common.h"

namespace moe {
namespace {

constexpr int kRowsPerBlock = 4;

template <bool BF16>
__global__ __launch_bounds__(256) void combine_kernel(const uint4* __restrict__ yp, const int32_t* __restrict__ inv,
                                                      const float* __restrict__ w, const uint4* __restrict__ ys,
                                                      int T, int k, int64_t row_chunks,
                                                      uint4* __restrict__ y) {
  const int t = blockIdx.x * kRowsPerBlock + (threadIdx.x >> 6);
  if (t >= T) return;
  const int lane = threadIdx.x & 63;
  const int P = T * k;
  int rows[kMaxK];
  float wt[kMaxK];
#pragma unroll
  for (int j = 0; j < kMaxK; ++j) {
    if (j >= k) break;
    int r = inv[static_cast<int64_t>(t) * k + j];
    // a negative entry marks a pair handled elsewhere: it adds nothing
    wt[j] = r < 0 ? 0.0f : w[static_cast<int64_t>(t) * k + j];
    rows[j] = r < 0 ? 0 : (r >= P ? P - 1 : r);
  }
  for (int64_t c = lane; c < row_chunks; c += 64) {
    constexpr int NE = BF16 ? 8 : 4;
    float acc[NE];
#pragma unroll
    for (int i = 0; i < NE; ++i) acc[i] = 0.0f;
#pragma unroll
    for (int j = 0; j < kMaxK; ++j) {
      if (j >= k) break;
      const uint4 v = yp[static_cast<int64_t>(rows[j]) * row_chunks + c];
      const uint32_t u[4] = {v.x, v.y, v.z, v.w};
      if (BF16) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          acc[2 * i] = fmaf(wt[j], __uint_as_float(u[i] << 16), acc[2 * i]);
          acc[2 * i + 1] = fmaf(wt[j], __uint_as_float(u[i] & 0xffff0000u), acc[2 * i + 1]);
        }
      } else {
#pragma unroll
        for (int i = 0; i < 4; ++i) acc[i] = fmaf(wt[j], __uint_as_float(u[i]), acc[i]);
      }
    }
    if (ys) {
      const uint4 v = ys[static_cast<int64_t>(t) * row_chunks + c];
      const uint32_t u[4] = {v.x, v.y, v.z, v.w};
      if (BF16) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          acc[2 * i] += __uint_as_float(u[i] << 16);
          acc[2 * i + 1] += __uint_as_float(u[i] & 0xffff0000u);
        }
      } else {
#pragma unroll
        for (int i = 0; i < 4; ++i) acc[i] += __uint_as_float(u[i]);
      }
    }
    uint4 o;
    if (BF16) {
      o.x = pack_bf16x2(acc[0], acc[1]);
      o.y = pack_bf16x2(acc[2], acc[3]);
      o.z = pack_bf16x2(acc[4], acc[5]);
      o.w = pack_bf16x2(acc[6], acc[7]);
    } else {
      o.x = __float_as_uint(acc[0]);
      o.y = __float_as_uint(acc[1]);
      o.z = __float_as_uint(acc[2]);
      o.w = __float_as_uint(acc[3]);
    }
    y[static_cast<int64_t>(t) * row_chunks + c] = o;
  }
}

}  // namespace
}  // namespace moe

using namespace moe;

extern "C" moe_status moe_unpermute_combine(const void* y_perm, const int32_t* inv_perm, const float* topk_w,
                                            const void* y_shared, int64_t T, int64_t d, int32_t k,
                                            moe_dtype dtype, void* y, void* stream) {
  if (T < 0 || d <= 0 || k < 1 || k > kMaxK || !valid_dtype(dtype)) return MOE_ERR_INVALID_ARG;
  if (d % 64 != 0) return MOE_ERR_ALIGNMENT;
  if (T * static_cast<int64_t>(k) >= (int64_t(1) << 31)) return MOE_ERR_UNSUPPORTED;
  if (T == 0) return MOE_OK;
  if (!y_perm || !inv_perm || !topk_w || !y) return MOE_ERR_INVALID_ARG;
  if (!aligned16(y_perm) || !aligned16(y) || (y_shared && !aligned16(y_shared))) return MOE_ERR_ALIGNMENT;
  const int64_t row_chunks = d * elem_bytes(dtype) / 16;
  const dim3 grid(static_cast<unsigned>(ceil_div(T, kRowsPerBlock)));
  hipStream_t st = as_stream(stream);
  if (dtype == MOE_BF16)
    hipLaunchKernelGGL(combine_kernel<true>, grid, dim3(256), 0, st, static_cast<const uint4*>(y_perm), inv_perm,
                       topk_w, static_cast<const uint4*>(y_shared), static_cast<int>(T), k, row_chunks,
                       static_cast<uint4*>(y));
  else
    hipLaunchKernelGGL(combine_kernel<false>, grid, dim3(256), 0, st, static_cast<const uint4*>(y_perm), inv_perm,
                       topk_w, static_cast<const uint4*>(y_shared), static_cast<int>(T), k, row_chunks,
                       static_cast<uint4*>(y));
  return launch_status();
}
