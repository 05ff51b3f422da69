// Small-batch (decode) expert projections: stream each active expert's
// weights from HBM once.
//
// The article "Mixture of Experts (MoEs) in Transformers" (section "From
// Dense to Sparse") estimates decode speed as memory bandwidth divided by
// the bytes of the active parameters; its section "Expert Backend" pairs
// small batches with a strategy that works per selected expert.  With a few
// tokens per expert the projection is a matrix-vector-like product whose
// cost is reading the weights, so the work is split along the weight rows
// of the experts that have tokens, and experts with no tokens are never
// read.
//
// Workgroup = (expert g, 16 output columns), 4 waves.  The K dimension is
// dealt to the waves in 32-element steps (wave w takes steps w, w+4, ...),
// so the workgroup streams each 16-row weight slab in 256-byte runs per row
// with many loads in flight; the four partial sums meet in LDS.  The tokens
// of the expert (up to 64 per pass) are the 16-wide operand of
// v_mfma_f32_16x16x32_bf16, the weight rows the 16-tall one, so each lane
// ends with 4 consecutive output columns of one token row.
#include "common.h"

namespace moe {
namespace {

constexpr int kMC = 4;        // 16-row token chunks per pass (64 tokens)

__device__ __forceinline__ bf16x8 ld8(const uint16_t* p) {
  return __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4*>(p));
}

template <bool SWIGLU>
__global__ __launch_bounds__(256) void decode_kernel(const uint16_t* __restrict__ A, const uint16_t* __restrict__ B,
                                                     const int32_t* __restrict__ off, int rows, int K, int N, int G,
                                                     uint16_t* __restrict__ C) {
  constexpr int NH = SWIGLU ? 2 : 1;
  __shared__ float red[4][kMC][NH][4][64];
  const int ntiles = N / 16;
  const int g = blockIdx.x / ntiles;
  if (g >= G) return;
  const int n0 = (blockIdx.x - g * ntiles) * 16;
  const int lo = clamp_off(off[g], rows);
  const int hi = clamp_off(off[g + 1], rows);
  if (hi <= lo) return;                      // expert without tokens: its weights are never read

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int i16 = lane & 15, kq = lane >> 4;
  const int64_t brows = SWIGLU ? 2 * static_cast<int64_t>(N) : N;
  const uint16_t* Bg = B + static_cast<int64_t>(g) * brows * K;
  const uint16_t* wg = Bg + static_cast<int64_t>(n0 + i16) * K + kq * 8;
  const uint16_t* wu = Bg + static_cast<int64_t>(SWIGLU ? N + n0 + i16 : n0 + i16) * K + kq * 8;
  const int steps = K / 32;
  const bf16x8 zero8 = __builtin_bit_cast(bf16x8, make_uint4(0, 0, 0, 0));

  for (int m0 = lo; m0 < hi; m0 += 16 * kMC) {
    const int mcn = min(kMC, (hi - m0 + 15) / 16);
    f32x4 ag[kMC], au[kMC];
    const uint16_t* xr[kMC];
    bool xv[kMC];
#pragma unroll
    for (int mc = 0; mc < kMC; ++mc) {
      ag[mc] = f32x4{};
      au[mc] = f32x4{};
      const int row = m0 + mc * 16 + i16;
      xv[mc] = (mc < mcn) && (row < hi);
      xr[mc] = A + static_cast<int64_t>(xv[mc] ? row : lo) * K + kq * 8;
    }
#pragma unroll 4
    for (int s = wave; s < steps; s += 4) {
      const int64_t k0 = static_cast<int64_t>(s) * 32;
      const bf16x8 wgf = ld8(wg + k0);
      bf16x8 wuf = zero8;
      if (SWIGLU) wuf = ld8(wu + k0);
#pragma unroll
      for (int mc = 0; mc < kMC; ++mc) {
        if (mc < mcn) {
          const bf16x8 tf = xv[mc] ? ld8(xr[mc] + k0) : zero8;
          ag[mc] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(wgf, tf, ag[mc], 0, 0, 0);
          if (SWIGLU) au[mc] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(wuf, tf, au[mc], 0, 0, 0);
        }
      }
    }
#pragma unroll
    for (int mc = 0; mc < kMC; ++mc) {
      if (mc < mcn) {
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          red[wave][mc][0][r][lane] = ag[mc][r];
          if (SWIGLU) red[wave][mc][NH - 1][r][lane] = au[mc][r];
        }
      }
    }
    __syncthreads();
    if (wave < mcn) {
      const int mc = wave;
      const int row = m0 + mc * 16 + i16;
      if (row < hi) {
        float o[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          float gs = red[0][mc][0][r][lane] + red[1][mc][0][r][lane] + red[2][mc][0][r][lane] +
                     red[3][mc][0][r][lane];
          if (SWIGLU) {
            const float us = red[0][mc][NH - 1][r][lane] + red[1][mc][NH - 1][r][lane] +
                             red[2][mc][NH - 1][r][lane] + red[3][mc][NH - 1][r][lane];
            gs = silu(gs) * us;
          }
          o[r] = gs;
        }
        uint2 v;
        v.x = pack_bf16x2(o[0], o[1]);
        v.y = pack_bf16x2(o[2], o[3]);
        *reinterpret_cast<uint2*>(C + static_cast<int64_t>(row) * N + n0 + 4 * kq) = v;
      }
    }
    __syncthreads();
  }
}

}  // namespace

moe_status decode_bf16(bool swiglu, const void* A, const void* B, const int32_t* off, int64_t rows, int64_t K,
                       int64_t N, int G, void* C, hipStream_t st) {
  const int64_t grid = static_cast<int64_t>(G) * (N / 16);
  if (grid > 0x7fffffff) return MOE_ERR_UNSUPPORTED;
  if (swiglu)
    hipLaunchKernelGGL(decode_kernel<true>, dim3(static_cast<unsigned>(grid)), dim3(256), 0, st,
                       static_cast<const uint16_t*>(A), static_cast<const uint16_t*>(B), off,
                       static_cast<int>(rows), static_cast<int>(K), static_cast<int>(N), G,
                       static_cast<uint16_t*>(C));
  else
    hipLaunchKernelGGL(decode_kernel<false>, dim3(static_cast<unsigned>(grid)), dim3(256), 0, st,
                       static_cast<const uint16_t*>(A), static_cast<const uint16_t*>(B), off,
                       static_cast<int>(rows), static_cast<int>(K), static_cast<int>(N), G,
                       static_cast<uint16_t*>(C));
  return launch_status();
}

}  // namespace moe
