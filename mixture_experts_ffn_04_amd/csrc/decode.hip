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
// Workgroup = (expert g, 16 output columns), 4 waves.  Each wave takes a
// contiguous quarter of K and streams it in unrolled batches (all loads of
// a batch issued before its MFMAs); the four partial sums meet in LDS.  The
// number of 16-token chunks (1, 2 or 4) is chosen per workgroup up front so
// the streaming loop itself has no branches.  The tokens of the expert (up
// to 64 per pass) are the 16-wide operand of v_mfma_f32_16x16x32_bf16, the
// weight rows the 16-tall one, so each lane ends with 4 consecutive output
// columns of one token row.
#include "common.h"

namespace moe {
namespace {

constexpr int kMC = 4;        // 16-row token chunks per pass (64 tokens)

typedef __attribute__((address_space(1))) const u32x4 gu4;

// 16-byte load of token rows and weight rows alike.  Token rows are reused
// by every weight tile of the expert.  Each weight load instruction touches
// whole 128-byte lines of its 16 rows (every other 16 bytes); the other step
// of the pair reads the rest from L2, so weights use cached loads too
// (non-temporal weight loads measured about 10% slower).
__device__ __forceinline__ bf16x8 ld8(const uint16_t* p) {
  return __builtin_bit_cast(bf16x8, *(const gu4*)p);
}

// K layout of a step: steps 2j and 2j+1 together cover elements
// [64j, 64j + 64) of every row; lane (row i, quarter q) holds elements
// 64j + 16q + [0, 8) in step 2j and 64j + 16q + [8, 16) in step 2j+1, so the
// two load instructions of a step pair each span whole 128-byte lines of the
// 16 rows (the row base pointers already include 16q).  Weights and tokens
// use the same layout, which only permutes the reduction over K.
__device__ __forceinline__ int64_t step_offset(int s) {
  return static_cast<int64_t>(s >> 1) * 64 + (s & 1) * 8;
}

// Partial sums of one wave over K steps [s0, s1) (32 elements each) for MC
// token chunks, in batches of U steps with every load of a batch issued
// before its MFMAs, so each wave keeps U x (NH + MC) 1 KB loads in flight.
// The last batch is padded: its steps past s1 load the last valid step and
// use a zero token fragment, so they add nothing and cost no extra round
// trip.
template <bool SWIGLU, int MC, int U>
__device__ __forceinline__ void decode_partial(const uint16_t* wg, const uint16_t* wu, const uint16_t* const* xr,
                                               int s0, int s1, f32x4* ag, f32x4* au) {
#pragma unroll
  for (int mc = 0; mc < MC; ++mc) {
    ag[mc] = f32x4{};
    au[mc] = f32x4{};
  }
  const bf16x8 zero8 = __builtin_bit_cast(bf16x8, u32x4{0u, 0u, 0u, 0u});
  for (int s = s0; s < s1; s += U) {
    bf16x8 wgf[U], wuf[U], tf[U][MC];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int su = s + u < s1 ? s + u : s1 - 1;
      const int64_t k0 = step_offset(su);
      wgf[u] = ld8(wg + k0);
      if (SWIGLU) wuf[u] = ld8(wu + k0);
#pragma unroll
      for (int mc = 0; mc < MC; ++mc) tf[u][mc] = ld8(xr[mc] + k0);
    }
    __builtin_amdgcn_sched_barrier(0);   // the whole batch of loads is issued before any MFMA waits
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const bool live = s + u < s1;
#pragma unroll
      for (int mc = 0; mc < MC; ++mc) {
        const bf16x8 t = live ? tf[u][mc] : zero8;
        ag[mc] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(wgf[u], t, ag[mc], 0, 0, 0);
        if (SWIGLU) au[mc] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(wuf[u], t, au[mc], 0, 0, 0);
      }
    }
  }
}

// EPI: 0 = bf16 store, 1 = SwiGLU pairs (bf16), 2 = fp32 + bias (router
// logits for small batches; N need not be a multiple of 16 there).
// rowmap (may be NULL): input row r is A[rowmap[r] / kdiv] (rowmap entries
// clamped to [0, rows)), the row gather of the sort folded into the loads.
template <int EPI>
__global__ __launch_bounds__(256) void decode_kernel(const uint16_t* __restrict__ A, const uint16_t* __restrict__ B,
                                                     const int32_t* __restrict__ off, const float* __restrict__ bias,
                                                     const int32_t* __restrict__ rowmap, int kdiv,
                                                     int rows, int K, int N, int G, int rb, void* __restrict__ Cv) {
  constexpr bool SWIGLU = EPI == 1;
  constexpr int NH = SWIGLU ? 2 : 1;
  __shared__ float red[4][kMC][NH][4][64];
  const int ntiles = (N + 15) / 16;
  const int j = blockIdx.x / ntiles;
  const int n0 = (blockIdx.x - j * ntiles) * 16;
  // compact grid: block row j is the j-th group that has rows
  const int g = (off && rows < G) ? nth_active_group(off, G, rows, j) : j;
  if (g < 0 || g >= G) return;
  int lo = off ? clamp_off(off[g], rows) : 0;
  int hi = off ? clamp_off(off[g + 1], rows) : rows;
  if (rb > 0) {                              // row split: this workgroup takes rows [lo + y*rb, +rb) of the group
    lo += static_cast<int>(blockIdx.y) * rb;
    hi = min(hi, lo + rb);
  }
  if (hi <= lo) return;                      // expert without tokens: its weights are never read

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int i16 = lane & 15, kq = lane >> 4;
  const int64_t brows = SWIGLU ? 2 * static_cast<int64_t>(N) : N;
  const uint16_t* Bg = B + static_cast<int64_t>(g) * brows * K;
  const int wrow = n0 + i16 < N ? n0 + i16 : N - 1;     // past-N rows read a valid row; never stored
  const uint16_t* wg = Bg + static_cast<int64_t>(wrow) * K + kq * 16;
  const uint16_t* wu = Bg + static_cast<int64_t>(SWIGLU ? N + wrow : wrow) * K + kq * 16;
  // contiguous K range per wave, in whole step pairs (K % 64 == 0)
  const int steps = K / 32;
  const int per = ((steps + 7) / 8) * 2;
  const int s0 = min(steps, wave * per);
  const int s1 = min(steps, s0 + per);

  for (int m0 = lo; m0 < hi; m0 += 16 * kMC) {
    const int mcn = min(kMC, (hi - m0 + 15) / 16);
    const uint16_t* xr[kMC];
    int src[kMC];
#pragma unroll
    for (int mc = 0; mc < kMC; ++mc) {
      const int row = m0 + mc * 16 + i16;        // rows past the group read a valid row; never stored
      src[mc] = row < hi ? row : lo;
    }
    if (rowmap) {                                // every map entry requested before any is used
      int rm[kMC];
#pragma unroll
      for (int mc = 0; mc < kMC; ++mc) rm[mc] = rowmap[src[mc]];
#pragma unroll
      for (int mc = 0; mc < kMC; ++mc) src[mc] = clamp_off(rm[mc], rows - 1) / kdiv;
    }
#pragma unroll
    for (int mc = 0; mc < kMC; ++mc) xr[mc] = A + static_cast<int64_t>(src[mc]) * K + kq * 16;
    f32x4 ag[kMC], au[kMC];
    if (mcn == 1) {
      decode_partial<SWIGLU, 1, 8>(wg, wu, xr, s0, s1, ag, au);
    } else if (mcn == 2) {
      decode_partial<SWIGLU, 2, 4>(wg, wu, xr, s0, s1, ag, au);
    } else {
      decode_partial<SWIGLU, 4, 4>(wg, wu, xr, s0, s1, ag, au);
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
        if (EPI == 2) {
          float* C = static_cast<float*>(Cv) + static_cast<int64_t>(row) * N;
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const int n = n0 + 4 * kq + r;
            if (n < N) C[n] = o[r] + (bias ? bias[n] : 0.0f);
          }
        } else {
          uint2 v;
          v.x = pack_bf16x2(o[0], o[1]);
          v.y = pack_bf16x2(o[2], o[3]);
          *reinterpret_cast<uint2*>(static_cast<uint16_t*>(Cv) + static_cast<int64_t>(row) * N + n0 + 4 * kq) = v;
        }
      }
    }
    __syncthreads();
  }
}

// rb > 0: the rows of each group are split into blocks of rb rows, one
// workgroup per (column tile, row block); gridDim.y covers the largest group.
template <int EPI>
moe_status launch_decode(const void* A, const void* B, const int32_t* off, const float* bias, const int32_t* rowmap,
                         int kdiv, int64_t rows, int64_t K, int64_t N, int G, void* C, hipStream_t st, int rb = 0) {
  if (off && G > 256) return MOE_ERR_UNSUPPORTED;                      // one group per thread
  const int64_t groups = off ? (G < rows ? G : rows) : G;             // at most `rows` groups have rows
  const int64_t grid = groups * ceil_div(N, 16);
  const int64_t gy = rb > 0 ? ceil_div(rows, rb) : 1;
  if (grid > 0x7fffffff || gy > 65535) return MOE_ERR_UNSUPPORTED;
  if (grid == 0 || gy == 0) return MOE_OK;
  hipLaunchKernelGGL(decode_kernel<EPI>, dim3(static_cast<unsigned>(grid), static_cast<unsigned>(gy)), dim3(256), 0, st,
                     static_cast<const uint16_t*>(A), static_cast<const uint16_t*>(B), off, bias, rowmap, kdiv,
                     static_cast<int>(rows), static_cast<int>(K), static_cast<int>(N), G, rb, C);
  return launch_status();
}

// ---------------------------------------------------------------------------
// Few rows per expert: dot products on the vector ALUs with row-contiguous
// loads.  With one or two tokens per expert the MFMA form above spends its
// loads on 16 rows x 64 bytes per instruction; here every load instruction
// reads 1 KB of one weight row, the pattern a plain streaming read uses
// (measured at T=1: gate/up 31.7 -> 26.0 us, down 18.2 -> 15.9 us; T=8:
// gate/up 121 -> 102 us, about 6 TB/s).  From four rows per expert on the
// MFMA form wins, since here every row costs one pass of dot products.
//
// Workgroup = (group, 8 weight rows), 4 waves with 2 rows each: the gate and
// up rows of one output column (SwiGLU) or two output columns.  Lane l
// holds 16-byte chunks l, l + 64, ... (at most CI) of both rows in
// registers, loaded once; each row of the group then costs CI
// v_dot2_f32_bf16 x 4 per weight row, a butterfly sum across the wave per
// weight row, and one store.  (Loading the next row's token chunks during
// the sums held 24 more VGPRs, one wave less per SIMD, and measured 2-5%
// slower at 1-6 rows per expert.)

template <int EPI, int CI>
__global__ __launch_bounds__(256) void decode_rows_kernel(const uint16_t* __restrict__ A, const uint16_t* __restrict__ B,
                                                          const int32_t* __restrict__ off,
                                                          const int32_t* __restrict__ rowmap, int kdiv,
                                                          int rows, int K, int N, int G, uint16_t* __restrict__ C) {
  constexpr bool SWIGLU = EPI == 1;
  constexpr int CPW = SWIGLU ? 1 : 2;                 // output columns per wave
  constexpr int CPB = 4 * CPW;                        // ... per workgroup
  const int ncb = (N + CPB - 1) / CPB;
  const int j = blockIdx.x / ncb;
  const int cb = blockIdx.x - j * ncb;
  const int g = (off && rows < G) ? nth_active_group(off, G, rows, j) : j;
  if (g < 0 || g >= G) return;
  const int lo = off ? clamp_off(off[g], rows) : 0;
  const int hi = off ? clamp_off(off[g + 1], rows) : rows;
  if (hi <= lo) return;                              // expert without tokens: its weights are never read
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int n0 = cb * CPB + wave * CPW;
  if (n0 >= N) return;                               // no barrier follows
  const int KC = K / 8;                              // 16-byte chunks per row
  const int64_t brows = SWIGLU ? 2 * static_cast<int64_t>(N) : N;
  const gu4* Bg = (const gu4*)B + static_cast<int64_t>(g) * brows * KC;
  // the wave's two weight rows: gate and up of column n0, or columns n0, n0+1
  const int r1 = SWIGLU ? N + n0 : (n0 + 1 < N ? n0 + 1 : n0);
  const gu4* w0p = Bg + static_cast<int64_t>(n0) * KC;
  const gu4* w1p = Bg + static_cast<int64_t>(r1) * KC;
  const u32x4 zero = {0u, 0u, 0u, 0u};
  auto token_row = [&](int m) {
    const int src = rowmap ? clamp_off(rowmap[m], rows - 1) / kdiv : m;
    return (const gu4*)A + static_cast<int64_t>(src) * KC;
  };
  // the first row's map entry is read before the weights, so its token
  // loads need not wait behind the weight loads (loads return in order)
  const gu4* xr_lo = token_row(lo);
  u32x4 w0[CI], w1[CI];
#pragma unroll
  for (int i = 0; i < CI; ++i) {
    const int c = lane + 64 * i;
    w0[i] = c < KC ? w0p[c] : zero;
    w1[i] = c < KC ? w1p[c] : zero;
  }
  for (int m = lo; m < hi; ++m) {
    const gu4* xr = m == lo ? xr_lo : token_row(m);
    u32x4 x[CI];
#pragma unroll
    for (int i = 0; i < CI; ++i) x[i] = (lane + 64 * i < KC) ? xr[lane + 64 * i] : zero;
    float a = 0.0f, b = 0.0f;
#pragma unroll
    for (int i = 0; i < CI; ++i) {
      a = dot8(w0[i], x[i], a);
      b = dot8(w1[i], x[i], b);
    }
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) {
      a += __shfl_xor(a, o, 64);
      b += __shfl_xor(b, o, 64);
    }
    if (lane == 0) {
      uint16_t* crow = C + static_cast<int64_t>(m) * N;
      if (SWIGLU) {
        crow[n0] = static_cast<uint16_t>(pack_bf16x2(silu(a) * b, 0.0f) & 0xffffu);
      } else {
        crow[n0] = static_cast<uint16_t>(pack_bf16x2(a, 0.0f) & 0xffffu);
        if (n0 + 1 < N) crow[n0 + 1] = static_cast<uint16_t>(pack_bf16x2(b, 0.0f) & 0xffffu);
      }
    }
  }
}

template <int EPI, int CI>
moe_status launch_decode_rows(const void* A, const void* B, const int32_t* off, const int32_t* rowmap, int kdiv,
                              int64_t rows, int64_t K, int64_t N, int G, void* C, hipStream_t st) {
  constexpr int CPB = (EPI == 1) ? 4 : 8;
  if (off && G > 256) return MOE_ERR_UNSUPPORTED;
  const int64_t groups = off ? (G < rows ? G : rows) : G;
  const int64_t grid = groups * ceil_div(N, CPB);
  if (grid > 0x7fffffff) return MOE_ERR_UNSUPPORTED;
  if (grid == 0) return MOE_OK;
  hipLaunchKernelGGL((decode_rows_kernel<EPI, CI>), dim3(static_cast<unsigned>(grid)), dim3(256), 0, st,
                     static_cast<const uint16_t*>(A), static_cast<const uint16_t*>(B), off, rowmap, kdiv,
                     static_cast<int>(rows), static_cast<int>(K), static_cast<int>(N), G, static_cast<uint16_t*>(C));
  return launch_status();
}

template <int EPI>
moe_status decode_rows(const void* A, const void* B, const int32_t* off, const int32_t* rowmap, int kdiv,
                       int64_t rows, int64_t K, int64_t N, int G, void* C, hipStream_t st) {
  if (K <= 2048) return launch_decode_rows<EPI, 4>(A, B, off, rowmap, kdiv, rows, K, N, G, C, st);
  if (K <= 3072) return launch_decode_rows<EPI, 6>(A, B, off, rowmap, kdiv, rows, K, N, G, C, st);
  return launch_decode_rows<EPI, 8>(A, B, off, rowmap, kdiv, rows, K, N, G, C, st);
}

}  // namespace

// At most two rows per expert on average (and K <= 4096, so a wave's rows
// fit its registers): the vector-ALU form; otherwise the MFMA form.
moe_status decode_bf16(bool swiglu, const void* A, const void* B, const int32_t* off, int64_t rows, int64_t K,
                       int64_t N, int G, void* C, hipStream_t st, const int32_t* rowmap, int kdiv) {
  if (rows <= 2 * static_cast<int64_t>(G) && K <= 4096)
    return swiglu ? decode_rows<1>(A, B, off, rowmap, kdiv, rows, K, N, G, C, st)
                  : decode_rows<0>(A, B, off, rowmap, kdiv, rows, K, N, G, C, st);
  return swiglu ? launch_decode<1>(A, B, off, nullptr, rowmap, kdiv, rows, K, N, G, C, st)
                : launch_decode<0>(A, B, off, nullptr, rowmap, kdiv, rows, K, N, G, C, st);
}

// Router logits for small batches: one group of T rows, N = E experts.
// rb > 0 splits the T rows over workgroups in blocks of rb.
moe_status decode_bf16_logits(const void* x, const void* w_router, const float* bias, int64_t T, int64_t d,
                              int32_t E, float* logits, hipStream_t st, int rb) {
  return launch_decode<2>(x, w_router, nullptr, bias, nullptr, 1, T, d, E, 1, logits, st, rb);
}

}  // namespace moe
