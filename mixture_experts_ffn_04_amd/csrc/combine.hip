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

// acc += wt * row chunk v (bf16: 8 values, fp32: 4)
template <bool BF16>
__device__ __forceinline__ void add_scaled(float (&acc)[8], const uint4& v, float wt) {
  const uint32_t u[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    if (BF16) {
      acc[2 * i] = fmaf(wt, __uint_as_float(u[i] << 16), acc[2 * i]);
      acc[2 * i + 1] = fmaf(wt, __uint_as_float(u[i] & 0xffff0000u), acc[2 * i + 1]);
    } else {
      acc[i] = fmaf(wt, __uint_as_float(u[i]), acc[i]);
    }
  }
}

template <bool BF16>
__device__ __forceinline__ void add_plain(float (&acc)[8], const uint4& v) {
  const uint32_t u[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    if (BF16) {
      acc[2 * i] += __uint_as_float(u[i] << 16);
      acc[2 * i + 1] += __uint_as_float(u[i] & 0xffff0000u);
    } else {
      acc[i] += __uint_as_float(u[i]);
    }
  }
}

// Streaming forms: the rows are read and the output written exactly once,
// so when they are far larger than the caches the non-temporal hint keeps
// them from evicting what is reused.
template <bool NT>
__device__ __forceinline__ uint4 load16(const uint4* p) {
  if (!NT) return *p;
  const u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
  return make_uint4(v[0], v[1], v[2], v[3]);
}

template <bool NT>
__device__ __forceinline__ void store16(uint4* p, const uint4& v) {
  if (!NT) {
    *p = v;
    return;
  }
  const u32x4 u = {v.x, v.y, v.z, v.w};
  __builtin_nontemporal_store(u, reinterpret_cast<u32x4*>(p));
}

template <bool BF16>
__device__ __forceinline__ uint4 pack_out(const float (&acc)[8]) {
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
  return o;
}

// KT > 0: k == KT is known at compile time, and each lane issues the loads
// of two column chunks of all k rows (and of the shared row) before any
// arithmetic, so 2k + 2 independent 16-byte loads per lane are in flight.
// KT == 0: any k, one chunk and one row at a time.  Both sum in the same
// order (increasing j, then the shared row), so they give identical bits.
// NT: non-temporal loads of the expert rows and stores of the output.
template <bool BF16, int KT, bool NT>
__global__ __launch_bounds__(256) void combine_kernel(const uint4* __restrict__ yp, const int32_t* __restrict__ inv,
                                                      const float* __restrict__ w, const uint4* __restrict__ ys,
                                                      int T, int k, int64_t row_chunks,
                                                      uint4* __restrict__ y) {
  const int t = blockIdx.x * kRowsPerBlock + (threadIdx.x >> 6);
  if (t >= T) return;
  const int lane = threadIdx.x & 63;
  const int kk = KT > 0 ? KT : k;
  const int P = T * kk;
  constexpr int KR = KT > 0 ? KT : kMaxK;
  int rows[KR];
  float wt[KR];
#pragma unroll
  for (int j = 0; j < KR; ++j) {
    if (KT == 0 && j >= kk) break;
    int r = inv[static_cast<int64_t>(t) * kk + j];
    // a negative entry marks a pair handled elsewhere: no row of y_perm is
    // read for it (y_perm may hold no written row at all), it adds zero
    wt[j] = r < 0 ? 0.0f : w[static_cast<int64_t>(t) * kk + j];
    rows[j] = r < 0 ? -1 : (r >= P ? P - 1 : r);
  }
  const uint4 zero = make_uint4(0u, 0u, 0u, 0u);
  const uint4* ysr = ys ? ys + static_cast<int64_t>(t) * row_chunks : nullptr;
  uint4* yr = y + static_cast<int64_t>(t) * row_chunks;
  if (KT > 0) {
    for (int64_t c0 = lane; c0 < row_chunks; c0 += 128) {
      const bool two = c0 + 64 < row_chunks;
      const int64_t c1 = two ? c0 + 64 : c0;       // a lone last chunk loads itself twice
      uint4 v0[KR], v1[KR], s0{}, s1{};
#pragma unroll
      for (int j = 0; j < KR; ++j) {
        v0[j] = rows[j] < 0 ? zero : load16<NT>(yp + static_cast<int64_t>(rows[j]) * row_chunks + c0);
        v1[j] = rows[j] < 0 ? zero : load16<NT>(yp + static_cast<int64_t>(rows[j]) * row_chunks + c1);
      }
      if (ysr) {
        s0 = ysr[c0];
        s1 = ysr[c1];
      }
      float a0[8] = {}, a1[8] = {};
#pragma unroll
      for (int j = 0; j < KR; ++j) {
        add_scaled<BF16>(a0, v0[j], wt[j]);
        add_scaled<BF16>(a1, v1[j], wt[j]);
      }
      if (ysr) {
        add_plain<BF16>(a0, s0);
        add_plain<BF16>(a1, s1);
      }
      store16<NT>(yr + c0, pack_out<BF16>(a0));
      if (two) store16<NT>(yr + c1, pack_out<BF16>(a1));
    }
  } else {
    for (int64_t c = lane; c < row_chunks; c += 64) {
      float acc[8] = {};
#pragma unroll
      for (int j = 0; j < KR; ++j) {
        if (j >= kk) break;
        add_scaled<BF16>(acc, rows[j] < 0 ? zero : load16<NT>(yp + static_cast<int64_t>(rows[j]) * row_chunks + c),
                         wt[j]);
      }
      if (ysr) add_plain<BF16>(acc, ysr[c]);
      store16<NT>(yr + c, pack_out<BF16>(acc));
    }
  }
}

// Expert rows beyond this many bytes are streamed with the non-temporal
// hint (measured: 1.9 GB of rows 475 -> 401 us; at 268 MB and below, where
// the rows the down projection just wrote are still partly in the 256 MB
// Infinity Cache, the hint measured slower).
constexpr int64_t kStreamCombineBytes = int64_t(512) << 20;

template <bool BF16, bool NT>
void launch_combine_nt(const void* y_perm, const int32_t* inv_perm, const float* topk_w, const void* y_shared,
                       int T, int k, int64_t row_chunks, void* y, hipStream_t st) {
  const dim3 grid(static_cast<unsigned>(ceil_div(T, kRowsPerBlock)));
  const uint4* yp = static_cast<const uint4*>(y_perm);
  const uint4* ys = static_cast<const uint4*>(y_shared);
  uint4* yo = static_cast<uint4*>(y);
#define MOE_COMBINE_K(KT_) \
  hipLaunchKernelGGL((combine_kernel<BF16, KT_, NT>), grid, dim3(256), 0, st, yp, inv_perm, topk_w, ys, T, k, row_chunks, yo)
  switch (k) {
    case 1: MOE_COMBINE_K(1); break;
    case 2: MOE_COMBINE_K(2); break;
    case 4: MOE_COMBINE_K(4); break;
    case 6: MOE_COMBINE_K(6); break;
    case 8: MOE_COMBINE_K(8); break;
    default: MOE_COMBINE_K(0); break;
  }
#undef MOE_COMBINE_K
}

template <bool BF16>
void launch_combine(const void* y_perm, const int32_t* inv_perm, const float* topk_w, const void* y_shared,
                    int T, int k, int64_t row_chunks, void* y, hipStream_t st) {
  if (static_cast<int64_t>(T) * k * row_chunks * 16 > kStreamCombineBytes)
    launch_combine_nt<BF16, true>(y_perm, inv_perm, topk_w, y_shared, T, k, row_chunks, y, st);
  else
    launch_combine_nt<BF16, false>(y_perm, inv_perm, topk_w, y_shared, T, k, row_chunks, y, st);
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
  if (dtype == MOE_BF16)
    launch_combine<true>(y_perm, inv_perm, topk_w, y_shared, static_cast<int>(T), k, row_chunks, y, as_stream(stream));
  else
    launch_combine<false>(y_perm, inv_perm, topk_w, y_shared, static_cast<int>(T), k, row_chunks, y, as_stream(stream));
  return launch_status();
}
