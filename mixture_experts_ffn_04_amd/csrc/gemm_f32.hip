// fp32 grouped GEMM (vector FMA, LDS-tiled) -- the fp32 element type of the
// layer.  Same grouping, schedule and epilogues as the bf16 MFMA kernel;
// every product and sum is an IEEE fp32 FMA.
//
// Tile: 64 token rows x 64 weight rows x 16 K, 256 threads, 4x4 outputs per
// thread.  The C tile goes through LDS so the SwiGLU epilogue can pair the
// gate column n (weight-tile row n) with the up column (row 32 + n).
#include "grouped_gemm.h"

namespace moe {

namespace {

constexpr int BM = 64, BN = 64, BK = 16;

template <int EPI>
__global__ __launch_bounds__(256) void gemm_f32_kernel(GemmArgs a) {
  constexpr int NT = 256;
  constexpr int BNO = (EPI == EPI_SWIGLU) ? BN / 2 : BN;
  __shared__ float sA[BK][BM + 4];
  __shared__ float sB[BK][BN + 4];
  __shared__ float sC[BM][BN + 1];

  TileLoc tl;
  if (!locate_tile<NT, BM, BNO, 4>(a, tl)) return;

  const int t = threadIdx.x;
  const int64_t K = a.K, N = a.N;
  const float* __restrict__ A = static_cast<const float*>(a.A);
  const float* __restrict__ B = static_cast<const float*>(a.B) +
      static_cast<int64_t>(tl.g) * ((EPI == EPI_SWIGLU) ? 2 * N : N) * K;

  // loader: 64 rows x 16 K per tile = 1024 floats = 4 per thread
  const int lr = t >> 2;            // row 0..63
  const int lk = (t & 3) * 4;       // k 0,4,8,12
  const int64_t arow = static_cast<int64_t>(tl.row0) + lr;
  const bool aok = arow < tl.row_end;
  int64_t brow;
  bool bok;
  if (EPI == EPI_SWIGLU) {
    const int half = lr / (BN / 2);
    const int64_t n = tl.n0 + (lr - half * (BN / 2));
    bok = n < N;
    brow = half * N + n;
  } else {
    const int64_t n = tl.n0 + lr;
    bok = n < N;
    brow = n;
  }
  const float* ap = A + (aok ? arow : 0) * K + lk;
  const float* bp = B + (bok ? brow : 0) * K + lk;

  const int tm = (t & 15) * 4;      // 4 token rows
  const int tn = (t >> 4) * 4;      // 4 weight rows
  float acc[4][4] = {};

  for (int64_t k0 = 0; k0 < K; k0 += BK) {
    float4 av = aok ? *reinterpret_cast<const float4*>(ap + k0) : make_float4(0, 0, 0, 0);
    float4 bv = bok ? *reinterpret_cast<const float4*>(bp + k0) : make_float4(0, 0, 0, 0);
    sA[lk + 0][lr] = av.x; sA[lk + 1][lr] = av.y; sA[lk + 2][lr] = av.z; sA[lk + 3][lr] = av.w;
    sB[lk + 0][lr] = bv.x; sB[lk + 1][lr] = bv.y; sB[lk + 2][lr] = bv.z; sB[lk + 3][lr] = bv.w;
    __syncthreads();
#pragma unroll
    for (int kk = 0; kk < BK; ++kk) {
      float x[4], w[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) { x[i] = sA[kk][tm + i]; w[i] = sB[kk][tn + i]; }
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = fmaf(x[i], w[j], acc[i][j]);
    }
    __syncthreads();
  }
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) sC[tm + i][tn + j] = acc[i][j];
  __syncthreads();

  float* C = static_cast<float*>(a.C);
  for (int idx = t; idx < BM * BNO; idx += NT) {
    const int r = idx / BNO, c = idx - r * BNO;
    const int64_t row = static_cast<int64_t>(tl.row0) + r;
    const int64_t n = tl.n0 + c;
    if (row >= tl.row_end || n >= N) continue;
    float v;
    if (EPI == EPI_SWIGLU) {
      const float g = sC[r][c], u = sC[r][BN / 2 + c];
      v = g / (1.0f + expf(-g)) * u;
    } else if (EPI == EPI_F32B) {
      v = sC[r][c] + (a.bias ? a.bias[n] : 0.0f);
    } else {
      v = sC[r][c];
    }
    C[row * N + n] = v;
  }
}

template <int EPI>
moe_status launch(const GemmArgs& a, hipStream_t st) {
  constexpr int BNO = (EPI == EPI_SWIGLU) ? BN / 2 : BN;
  const int64_t grid = grouped_tile_bound(a.rows, a.G, BM, a.N, BNO);
  if (grid <= 0) return MOE_OK;
  if (grid > 0x7fffffff) return MOE_ERR_UNSUPPORTED;
  hipLaunchKernelGGL((gemm_f32_kernel<EPI>), dim3(static_cast<unsigned>(grid)), dim3(256), 0, st, a);
  return launch_status();
}

}  // namespace

moe_status gemm_f32_gateup_swiglu(const GemmArgs& a, hipStream_t st) { return launch<EPI_SWIGLU>(a, st); }
moe_status gemm_f32_down(const GemmArgs& a, hipStream_t st) { return launch<EPI_STORE>(a, st); }
moe_status gemm_f32_logits(const GemmArgs& a, hipStream_t st) { return launch<EPI_F32B>(a, st); }

}  // namespace moe
