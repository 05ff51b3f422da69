// Decode-sized expert projections with MXFP4 expert weights and bf16
// activations, fp32 accumulation.
//
// The article "Mixture of Experts (MoEs) in Transformers" (section "From
// Dense to Sparse") notes that decoding would be faster still with kernels
// for the native mxfp4 format of gpt-oss's experts: decode streams the
// active experts' weights, and MXFP4 stores them in 4.25 bits per element.
// The format is the OCP Microscaling (MX) v1.0 one: blocks of 32 E2M1
// elements (two per byte, element 2i in the low nibble) sharing one E8M0
// scale X = 2^(s - 127); an element's value is X times its E2M1 value.
//
// Workgroup = (expert g with rows, CPB output columns), 4 waves; each wave
// owns R = 4 weight rows (gate/up: the gate and up rows of 2 columns; down:
// 4 columns).  Lane l keeps blocks l, l + 64, ... of its 4 rows in
// registers (16 code bytes and one scale per block), loaded once: the
// expert's weights are read from HBM once.  Then for every token row of the
// expert, the lane loads the 64 bytes of activations under each of its
// blocks, turns each code byte into two bf16 values
// (v_cvt_scalef32_pk_bf16_fp4 with scale 1: E2M1 values are exact in
// bf16), takes their dot product with the activations (v_dot2_f32_bf16),
// multiplies the block's sum by its scale (a power of two, exact in fp32
// for scale codes 1..254 short of overflow) and the wave sums its lanes.
// Experts without rows are never read.
#include "common.h"
#include "select.h"

namespace moe {
namespace {

typedef __attribute__((address_space(1))) const u32x4 gu4;
typedef __bf16 bf16x2v __attribute__((ext_vector_type(2)));

constexpr int kMxRows = 4;            // weight rows per wave
constexpr int64_t kMxMaxRows = 1024;  // routed rows per call (decode sizes)
// Above this many rows per expert on average the split-K MFMA form runs:
// the vector form re-reads each activation row for every 4 weight rows.
constexpr int64_t kMxVectorRowsPerExpert = 1;

// Elements 2B and 2B + 1 of a code dword (byte B) as bf16, times x's pair.
template <int B>
__device__ __forceinline__ float byte_dot(uint32_t qd, uint32_t xp, float s) {
  const bf16x2v w2 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(qd, 1.0f, B);
  return dot2(__builtin_bit_cast(uint32_t, w2), xp, s);
}

// sum over the 32 elements of one block: codes (16 bytes) . x (32 bf16);
// code dword dw holds elements 8 dw .. 8 dw + 7, as does x[dw]
__device__ __forceinline__ float block_dot(const u32x4& q, const u32x4 (&x)[4]) {
  float s = 0.0f;
#pragma unroll
  for (int dw = 0; dw < 4; ++dw) {
    s = byte_dot<0>(q[dw], x[dw][0], s);
    s = byte_dot<1>(q[dw], x[dw][1], s);
    s = byte_dot<2>(q[dw], x[dw][2], s);
    s = byte_dot<3>(q[dw], x[dw][3], s);
  }
  return s;
}

// The codes and scale codes of the kMxRows weight rows wr[] of one expert
// (Bqg, Bsg: its codes [rows][K/2] and scales [rows][K/32]): lane l holds
// blocks l, l + 64, ... (CI of them).  The scale codes stay raw bytes here
// and are decoded where they are used, so no load waits for an earlier
// one's data before it is issued.
template <int CI>
__device__ __forceinline__ void mx_load_rows(const uint8_t* Bqg, const uint8_t* Bsg, const int (&wr)[kMxRows], int K,
                                             int KB, int lane, u32x4 (&wq)[kMxRows][CI], uint32_t (&ws)[kMxRows][CI]) {
  const u32x4 zero = {0u, 0u, 0u, 0u};
#pragma unroll
  for (int r = 0; r < kMxRows; ++r) {
#pragma unroll
    for (int i = 0; i < CI; ++i) {
      const int b = lane + 64 * i;
      const bool ok = b < KB;
      wq[r][i] = ok ? *(const gu4*)(Bqg + static_cast<int64_t>(wr[r]) * (K / 2) + b * 16) : zero;
      ws[r][i] = ok ? Bsg[static_cast<int64_t>(wr[r]) * KB + b] : 0u;
    }
  }
}

// The 64 bytes of activation row xr (bf16, K long) under each of the
// lane's blocks.
template <int CI>
__device__ __forceinline__ void mx_load_x(const uint16_t* xr, int KB, int lane, u32x4 (&xv)[CI][4]) {
  const u32x4 zero = {0u, 0u, 0u, 0u};
#pragma unroll
  for (int i = 0; i < CI; ++i) {
    const int b = lane + 64 * i;
#pragma unroll
    for (int c = 0; c < 4; ++c) xv[i][c] = b < KB ? *(const gu4*)(xr + b * 32 + c * 8) : zero;
  }
}

// The wave's dot products of one activation row (xv, from mx_load_x) with
// its kMxRows weight rows, in every lane: per lane, each block's sum times
// the block's scale, accumulated over the lane's blocks in order, then
// summed across the wave.
template <int CI>
__device__ __forceinline__ void mx_dot_rows(const u32x4 (&wq)[kMxRows][CI], const uint32_t (&ws)[kMxRows][CI],
                                            const u32x4 (&xv)[CI][4], int KB, int lane, float (&acc)[kMxRows]) {
#pragma unroll
  for (int r = 0; r < kMxRows; ++r) acc[r] = 0.0f;
#pragma unroll
  for (int i = 0; i < CI; ++i) {
    if (lane + 64 * i < KB) {
#pragma unroll
      for (int r = 0; r < kMxRows; ++r) acc[r] = fmaf(block_dot(wq[r][i], xv[i]), e8m0_to_f32(ws[r][i]), acc[r]);
    }
  }
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) {
#pragma unroll
    for (int r = 0; r < kMxRows; ++r) acc[r] += __shfl_xor(acc[r], o, 64);
  }
}

// The wave's outputs (lane 0 stores them at crow): SwiGLU of rows (0, 2)
// and (1, 3) -- the gate and up rows of two columns -- or the four rows.
template <bool SWIGLU>
__device__ __forceinline__ void mx_store(const float (&acc)[kMxRows], int lane, uint16_t* crow) {
  if (lane != 0) return;
  if (SWIGLU) {
    *reinterpret_cast<uint32_t*>(crow) = pack_bf16x2(silu(acc[0]) * acc[2], silu(acc[1]) * acc[3]);
  } else {
    uint2 v;
    v.x = pack_bf16x2(acc[0], acc[1]);
    v.y = pack_bf16x2(acc[2], acc[3]);
    *reinterpret_cast<uint2*>(crow) = v;
  }
}

// Weight rows of the wave's output columns n0, n0 + 1 (SwiGLU: gate rows n0,
// n0 + 1 and up rows N + n0, N + n0 + 1) or n0 .. n0 + 3.
template <bool SWIGLU>
__device__ __forceinline__ void mx_wave_rows(int n0, int N, int (&wr)[kMxRows]) {
#pragma unroll
  for (int r = 0; r < kMxRows; ++r) wr[r] = SWIGLU ? (r < 2 ? n0 + r : N + n0 + r - 2) : n0 + r;
}

// SWIGLU: C = h [rows][N], B = gate/up [G][2N][K/2] codes + [G][2N][K/32]
// scales; else C = y_perm [rows][N], B = down [G][N][K/2] + [G][N][K/32].
// A: activation rows [.][K] bf16; with rowmap, row r reads A[rowmap[r] /
// kdiv] (rowmap entries clamped to [0, rows)).
template <bool SWIGLU, int CI>
__global__ __launch_bounds__(256) void decode_mx_kernel(const uint16_t* __restrict__ A, const uint8_t* __restrict__ Bq,
                                                        const uint8_t* __restrict__ Bs, const int32_t* __restrict__ off,
                                                        const int32_t* __restrict__ rowmap, int kdiv, int rows, int K,
                                                        int N, int G, uint16_t* __restrict__ C) {
  constexpr int CPW = SWIGLU ? kMxRows / 2 : kMxRows;   // output columns per wave
  constexpr int CPB = 4 * CPW;                           // ... per workgroup
  const int ncb = N / CPB;
  const int j = blockIdx.x / ncb;
  const int cb = blockIdx.x - j * ncb;
  const int g = (rows < G) ? nth_active_group(off, G, rows, j) : j;
  if (g < 0 || g >= G) return;
  const int lo = clamp_off(off[g], rows);
  const int hi = clamp_off(off[g + 1], rows);
  if (hi <= lo) return;                                  // expert without rows: its weights are never read
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int n0 = cb * CPB + wave * CPW;
  const int KB = K / 32;                                 // blocks per row
  const int64_t brows = SWIGLU ? 2 * static_cast<int64_t>(N) : N;
  int wr[kMxRows];
  mx_wave_rows<SWIGLU>(n0, N, wr);
  // the first row's map entry is read before the weights, so its
  // activation loads need not wait behind the code loads (loads return in
  // order)
  const int src_lo = rowmap ? clamp_off(rowmap[lo], rows - 1) / kdiv : lo;
  u32x4 wq[kMxRows][CI];
  uint32_t ws[kMxRows][CI];
  mx_load_rows<CI>(Bq + static_cast<int64_t>(g) * brows * (K / 2), Bs + static_cast<int64_t>(g) * brows * KB, wr, K,
                   KB, lane, wq, ws);
  // the first row's activations are requested right behind the codes
  u32x4 xv[CI][4];
  mx_load_x<CI>(A + static_cast<int64_t>(src_lo) * K, KB, lane, xv);
  for (int m = lo; m < hi; ++m) {
    if (m > lo) {
      const int src = rowmap ? clamp_off(rowmap[m], rows - 1) / kdiv : m;
      mx_load_x<CI>(A + static_cast<int64_t>(src) * K, KB, lane, xv);
    }
    float acc[kMxRows];
    mx_dot_rows<CI>(wq, ws, xv, KB, lane, acc);
    mx_store<SWIGLU>(acc, lane, C + static_cast<int64_t>(m) * N + n0);
  }
}

// ---------------------------------------------------------------------------
// The "batched_mm" strategy with MXFP4 experts (the article's section
// "Expert Backend"): every (token, slot) pair p multiplies the weights of
// its expert ids[p] in place, with no sort; the down call applies the
// routing weights and sums a token's slots.  The per-row arithmetic is that
// of decode_mx_kernel, so a pair's h row equals the one the decode call's
// vector form computes, bit for bit.

// h[p][n] for p < P: workgroup = (pair p, 8 output columns), two per wave.
// S > 0: the experts are selected here from the router logits [T][E] (every
// wave runs its token's selection), and the first workgroup of each token
// writes the token's ids and weights.
template <int CI, int S>
__global__ __launch_bounds__(256) void batched_mx_gateup_kernel(const uint16_t* __restrict__ x,
                                                                int32_t* __restrict__ ids,
                                                                const float* __restrict__ logits, int score,
                                                                float* __restrict__ wts,
                                                                const uint8_t* __restrict__ Bq,
                                                                const uint8_t* __restrict__ Bs, int P, int k, int E,
                                                                int K, int N, uint16_t* __restrict__ h) {
  constexpr int CPW = kMxRows / 2, CPB = 4 * CPW;
  const int ncb = N / CPB;
  const int p = blockIdx.x / ncb;
  const int cb = blockIdx.x - p * ncb;
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
  if (e < 0 || e >= E) return;                           // a pair of an expert held elsewhere
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int n0 = cb * CPB + wave * CPW;
  const int KB = K / 32;
  int wr[kMxRows];
  mx_wave_rows<true>(n0, N, wr);
  u32x4 wq[kMxRows][CI];
  uint32_t ws[kMxRows][CI];
  mx_load_rows<CI>(Bq + static_cast<int64_t>(e) * 2 * N * (K / 2), Bs + static_cast<int64_t>(e) * 2 * N * KB, wr, K,
                   KB, lane, wq, ws);
  u32x4 xv[CI][4];
  mx_load_x<CI>(x + static_cast<int64_t>(p / k) * K, KB, lane, xv);
  float acc[kMxRows];
  mx_dot_rows<CI>(wq, ws, xv, KB, lane, acc);
  mx_store<true>(acc, lane, h + static_cast<int64_t>(p) * N + n0);
}

// y[t][c] = sum_j w[t][j] * (h[t*k+j] . Wd[e_tj][c])  (+ y_shared[t][c]),
// in fp32 in increasing j, then the shared row, rounded once.  Workgroup =
// (token t, 4 output columns); wave w takes slots j = w, w + 4, ..., each
// slot's four dot products go to LDS, and one thread per column sums them
// in slot order.  Slots with an id outside [0, E) add nothing.
template <int CI>
__global__ __launch_bounds__(256) void batched_mx_down_combine_kernel(
    const uint16_t* __restrict__ h, const int32_t* __restrict__ ids, const float* __restrict__ wts,
    const uint8_t* __restrict__ Bq, const uint8_t* __restrict__ Bs, const uint16_t* __restrict__ ys, int T, int k,
    int E, int K, int N, uint16_t* __restrict__ y) {
  __shared__ float part[kMaxK][kMxRows];
  const int ncb = N / kMxRows;
  const int t = blockIdx.x / ncb;
  const int c0 = (blockIdx.x - t * ncb) * kMxRows;
  if (t >= T) return;                                    // uniform over the workgroup
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int KB = K / 32;
  for (int j = wave; j < k; j += 4) {
    const int64_t p = static_cast<int64_t>(t) * k + j;
    const int e = ids[p];
    float acc[kMxRows] = {};
    if (e >= 0 && e < E) {
      int wr[kMxRows];
      mx_wave_rows<false>(c0, N, wr);
      u32x4 wq[kMxRows][CI];
      uint32_t ws[kMxRows][CI];
      mx_load_rows<CI>(Bq + static_cast<int64_t>(e) * N * (K / 2), Bs + static_cast<int64_t>(e) * N * KB, wr, K, KB,
                       lane, wq, ws);
      u32x4 xv[CI][4];
      mx_load_x<CI>(h + p * K, KB, lane, xv);
      mx_dot_rows<CI>(wq, ws, xv, KB, lane, acc);
    }
    if (lane == 0) {
#pragma unroll
      for (int r = 0; r < kMxRows; ++r) part[j][r] = acc[r];
    }
  }
  __syncthreads();
  if (threadIdx.x < kMxRows) {
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

// ---------------------------------------------------------------------------
// Several rows per expert: the split-K MFMA form (v_mfma_f32_16x16x32_bf16,
// weight rows as the 16-row operand, tokens as the 16-column one).
//
// K is walked in quads of 128 elements.  In quad j, lane (row i = lane % 16,
// part q = lane / 16) holds elements 128j + 32q + [0, 32) of its row: one
// whole MX block, so a single 16-byte load brings its codes and one byte its
// scale.  MFMA m (0..3) of the quad takes elements 128j + 32q + 8m + [0, 8)
// from every lane, of the weights and of the tokens alike, which only
// permutes the order of the reduction over K.  The gfx950 FP4 conversion
// applies the block's power of two while decoding, so the bf16 operand is
// the weight's value.  A last half quad (K % 128 == 64) leaves parts 2 and 3
// without elements: their weights and tokens load as zeros.
//
// Workgroup = (expert g, 16 output columns), 4 waves splitting the quads;
// each wave issues all loads of a batch of U quads before its MFMAs; the
// four partial sums meet in LDS.
template <bool SWIGLU, int MC, int U>
__device__ __forceinline__ void mx_partial(const uint8_t* wq_g, const uint8_t* ws_g, const uint8_t* wq_u,
                                           const uint8_t* ws_u, const uint16_t* const* xr, int q0, int q1, int part,
                                           int KB, f32x4* ag, f32x4* au) {
  typedef __bf16 b2 __attribute__((ext_vector_type(2)));
#pragma unroll
  for (int mc = 0; mc < MC; ++mc) {
    ag[mc] = f32x4{};
    au[mc] = f32x4{};
  }
  const u32x4 zero = {0u, 0u, 0u, 0u};
  for (int qb = q0; qb < q1; qb += U) {
    u32x4 cg[U], cu[U], tk[U][MC][4];
    uint32_t sg[U], su[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int b = (qb + u) * 4 + part;             // this lane's block
      const bool ok = qb + u < q1 && b < KB;
      cg[u] = ok ? *(const gu4*)(wq_g + b * 16) : zero;
      sg[u] = ok ? ws_g[b] : 127u;
      if (SWIGLU) {
        cu[u] = ok ? *(const gu4*)(wq_u + b * 16) : zero;
        su[u] = ok ? ws_u[b] : 127u;
      }
#pragma unroll
      for (int mc = 0; mc < MC; ++mc)
#pragma unroll
        for (int c = 0; c < 4; ++c) tk[u][mc][c] = ok ? *(const gu4*)(xr[mc] + b * 32 + c * 8) : zero;
    }
    __builtin_amdgcn_sched_barrier(0);   // the whole batch of loads is issued before any MFMA waits
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const float xg = e8m0_to_f32(sg[u]);
      const float xu = SWIGLU ? e8m0_to_f32(su[u]) : 0.0f;
#pragma unroll
      for (int m = 0; m < 4; ++m) {
        u32x4 wg, wu;
        wg[0] = __builtin_bit_cast(uint32_t, (b2)__builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(cg[u][m], xg, 0));
        wg[1] = __builtin_bit_cast(uint32_t, (b2)__builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(cg[u][m], xg, 1));
        wg[2] = __builtin_bit_cast(uint32_t, (b2)__builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(cg[u][m], xg, 2));
        wg[3] = __builtin_bit_cast(uint32_t, (b2)__builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(cg[u][m], xg, 3));
        if (SWIGLU) {
          wu[0] = __builtin_bit_cast(uint32_t, (b2)__builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(cu[u][m], xu, 0));
          wu[1] = __builtin_bit_cast(uint32_t, (b2)__builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(cu[u][m], xu, 1));
          wu[2] = __builtin_bit_cast(uint32_t, (b2)__builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(cu[u][m], xu, 2));
          wu[3] = __builtin_bit_cast(uint32_t, (b2)__builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(cu[u][m], xu, 3));
        }
#pragma unroll
        for (int mc = 0; mc < MC; ++mc) {
          const bf16x8 t = __builtin_bit_cast(bf16x8, tk[u][mc][m]);
          ag[mc] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, wg), t, ag[mc], 0, 0, 0);
          if (SWIGLU)
            au[mc] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, wu), t, au[mc], 0, 0, 0);
        }
      }
    }
  }
}

template <bool SWIGLU>
__global__ __launch_bounds__(256) void decode_mx_mfma_kernel(const uint16_t* __restrict__ A,
                                                             const uint8_t* __restrict__ Bq,
                                                             const uint8_t* __restrict__ Bs,
                                                             const int32_t* __restrict__ off,
                                                             const int32_t* __restrict__ rowmap, int kdiv, int rows,
                                                             int K, int N, int G, uint16_t* __restrict__ C) {
  constexpr int MCX = 4;                              // 16-token chunks per pass (64 tokens)
  constexpr int NH = SWIGLU ? 2 : 1;
  __shared__ float red[4][MCX][NH][4][64];
  const int ntiles = N / 16;
  const int j = blockIdx.x / ntiles;
  const int n0 = (blockIdx.x - j * ntiles) * 16;
  const int g = (rows < G) ? nth_active_group(off, G, rows, j) : j;
  if (g < 0 || g >= G) return;
  const int lo = clamp_off(off[g], rows);
  const int hi = clamp_off(off[g + 1], rows);
  if (hi <= lo) return;                               // expert without rows: its weights are never read
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int i16 = lane & 15, part = lane >> 4;
  const int KB = K / 32;
  const int64_t brows = SWIGLU ? 2 * static_cast<int64_t>(N) : N;
  const int64_t wrow = n0 + i16;                      // N is a multiple of 16: always a valid row
  const int64_t urow = SWIGLU ? N + wrow : wrow;
  const uint8_t* Bqg = Bq + static_cast<int64_t>(g) * brows * (K / 2);
  const uint8_t* Bsg = Bs + static_cast<int64_t>(g) * brows * KB;
  const uint8_t* wq_g = Bqg + wrow * (K / 2);
  const uint8_t* wq_u = Bqg + urow * (K / 2);
  const uint8_t* ws_g = Bsg + wrow * KB;
  const uint8_t* ws_u = Bsg + urow * KB;
  // contiguous quads per wave
  const int quads = (KB + 3) / 4;
  const int per = (quads + 3) / 4;
  const int q0 = min(quads, wave * per);
  const int q1 = min(quads, q0 + per);
  for (int m0 = lo; m0 < hi; m0 += 16 * MCX) {
    const int mcn = min(MCX, (hi - m0 + 15) / 16);
    const uint16_t* xr[MCX];
    int src[MCX];
#pragma unroll
    for (int mc = 0; mc < MCX; ++mc) {
      const int row = m0 + mc * 16 + i16;             // rows past the group read a valid row; never stored
      src[mc] = row < hi ? row : lo;
    }
    if (rowmap) {                                     // every map entry requested before any is used
      int rm[MCX];
#pragma unroll
      for (int mc = 0; mc < MCX; ++mc) rm[mc] = rowmap[src[mc]];
#pragma unroll
      for (int mc = 0; mc < MCX; ++mc) src[mc] = clamp_off(rm[mc], rows - 1) / kdiv;
    }
#pragma unroll
    for (int mc = 0; mc < MCX; ++mc) xr[mc] = A + static_cast<int64_t>(src[mc]) * K;
    f32x4 ag[MCX], au[MCX];
    if (mcn == 1) {
      mx_partial<SWIGLU, 1, 4>(wq_g, ws_g, wq_u, ws_u, xr, q0, q1, part, KB, ag, au);
    } else if (mcn == 2) {
      mx_partial<SWIGLU, 2, 2>(wq_g, ws_g, wq_u, ws_u, xr, q0, q1, part, KB, ag, au);
    } else {
      mx_partial<SWIGLU, 4, 1>(wq_g, ws_g, wq_u, ws_u, xr, q0, q1, part, KB, ag, au);
    }
#pragma unroll
    for (int mc = 0; mc < MCX; ++mc) {
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
        *reinterpret_cast<uint2*>(C + static_cast<int64_t>(row) * N + n0 + 4 * part) = v;
      }
    }
    __syncthreads();
  }
}

template <bool SWIGLU>
moe_status launch_mx_mfma(const void* A, const void* Bq, const void* Bs, const int32_t* off, const int32_t* rowmap,
                          int kdiv, int64_t rows, int64_t K, int64_t N, int G, void* C, hipStream_t st) {
  const int64_t groups = G < rows ? G : rows;
  const int64_t grid = groups * (N / 16);
  if (grid == 0) return MOE_OK;
  if (grid > 0x7fffffff) return MOE_ERR_UNSUPPORTED;
  hipLaunchKernelGGL((decode_mx_mfma_kernel<SWIGLU>), dim3(static_cast<unsigned>(grid)), dim3(256), 0, st,
                     static_cast<const uint16_t*>(A), static_cast<const uint8_t*>(Bq), static_cast<const uint8_t*>(Bs),
                     off, rowmap, kdiv, static_cast<int>(rows), static_cast<int>(K), static_cast<int>(N), G,
                     static_cast<uint16_t*>(C));
  return launch_status();
}

template <bool SWIGLU>
moe_status launch_mx(const void* A, const void* Bq, const void* Bs, const int32_t* off, const int32_t* rowmap,
                     int kdiv, int64_t rows, int64_t K, int64_t N, int G, void* C, hipStream_t st) {
  constexpr int CPB = 4 * (SWIGLU ? kMxRows / 2 : kMxRows);
  const int64_t groups = G < rows ? G : rows;            // at most `rows` experts have rows
  const int64_t grid = groups * (N / CPB);
  if (grid == 0) return MOE_OK;
  if (grid > 0x7fffffff) return MOE_ERR_UNSUPPORTED;
  const int KB = static_cast<int>(K / 32);
#define MOE_MX_LAUNCH(CI_)                                                                                    \
  hipLaunchKernelGGL((decode_mx_kernel<SWIGLU, CI_>), dim3(static_cast<unsigned>(grid)), dim3(256), 0, st,      \
                     static_cast<const uint16_t*>(A), static_cast<const uint8_t*>(Bq),                         \
                     static_cast<const uint8_t*>(Bs), off, rowmap, kdiv, static_cast<int>(rows),               \
                     static_cast<int>(K), static_cast<int>(N), G, static_cast<uint16_t*>(C))
  if (KB <= 64) MOE_MX_LAUNCH(1);
  else if (KB <= 128) MOE_MX_LAUNCH(2);
  else MOE_MX_LAUNCH(4);
#undef MOE_MX_LAUNCH
  return launch_status();
}

moe_status check_mx(const void* in, const void* wq, const void* ws, const int32_t* offsets, int64_t rows, int64_t d,
                    int64_t f, int32_t E, const void* out, int64_t K) {
  if (rows < 0 || d <= 0 || f <= 0 || E < 1) return MOE_ERR_INVALID_ARG;
  if (E > kMaxE || rows > kMxMaxRows || K > 8192) return MOE_ERR_UNSUPPORTED;
  if (d % 64 != 0 || f % 64 != 0) return MOE_ERR_ALIGNMENT;
  if (rows == 0) return MOE_OK;
  if (!in || !wq || !ws || !offsets || !out) return MOE_ERR_INVALID_ARG;
  if (!aligned16(in) || !aligned16(wq) || !aligned16(out)) return MOE_ERR_ALIGNMENT;
  return MOE_OK;
}

constexpr int64_t kMxBatchedMaxPairs = 1024;

moe_status check_batched_mx(const void* in, const int32_t* ids, const void* wq, const void* ws, int64_t T, int64_t d,
                            int64_t f, int32_t E, int32_t k, const void* out) {
  if (T < 0 || d <= 0 || f <= 0 || E < 1 || k < 1 || k > kMaxK) return MOE_ERR_INVALID_ARG;
  if (E > kMaxE || T * k > kMxBatchedMaxPairs || d > 8192 || f > 8192) return MOE_ERR_UNSUPPORTED;
  if (d % 64 != 0 || f % 64 != 0) return MOE_ERR_ALIGNMENT;
  if (T == 0) return MOE_OK;
  if (!in || !ids || !wq || !ws || !out) return MOE_ERR_INVALID_ARG;
  if (!aligned16(in) || !aligned16(wq)) return MOE_ERR_ALIGNMENT;
  return MOE_OK;
}

}  // namespace
}  // namespace moe

using namespace moe;

extern "C" moe_status moe_batched_gateup_swiglu_mxfp4(const void* x, const int32_t* topk_ids, const void* wq_gate_up,
                                                      const void* ws_gate_up, int64_t T, int64_t d, int64_t f,
                                                      int32_t E, int32_t k, void* h, void* stream) {
  moe_status s = check_batched_mx(x, topk_ids, wq_gate_up, ws_gate_up, T, d, f, E, k, h);
  if (s != MOE_OK || T == 0) return s;
  const int64_t P = T * k;
  const int KB = static_cast<int>(d / 32);
  const dim3 grid(static_cast<unsigned>(P * (f / (2 * kMxRows))));
#define MOE_BMX_GU(CI_)                                                                                          \
  hipLaunchKernelGGL((batched_mx_gateup_kernel<CI_, 0>), grid, dim3(256), 0, as_stream(stream),                  \
                     static_cast<const uint16_t*>(x), const_cast<int32_t*>(topk_ids), nullptr, 0, nullptr,       \
                     static_cast<const uint8_t*>(wq_gate_up), static_cast<const uint8_t*>(ws_gate_up),           \
                     static_cast<int>(P), k, E, static_cast<int>(d), static_cast<int>(f), static_cast<uint16_t*>(h))
  if (KB <= 64) MOE_BMX_GU(1);
  else if (KB <= 128) MOE_BMX_GU(2);
  else MOE_BMX_GU(4);
#undef MOE_BMX_GU
  return launch_status();
}

extern "C" moe_status moe_batched_gateup_swiglu_mxfp4_select(const void* x, const float* logits,
                                                             const void* wq_gate_up, const void* ws_gate_up,
                                                             int64_t T, int64_t d, int64_t f, int32_t E, int32_t k,
                                                             moe_score score, int32_t* topk_ids, float* topk_w,
                                                             void* h, void* stream) {
  moe_status s = check_batched_mx(x, logits ? topk_ids : nullptr, wq_gate_up, ws_gate_up, T, d, f, E, k, h);
  if (s != MOE_OK || T == 0) return s;
  if (!topk_w || k > E || (score != MOE_SCORE_SOFTMAX && score != MOE_SCORE_SIGMOID)) return MOE_ERR_INVALID_ARG;
  const int64_t P = T * k;
  const int KB = static_cast<int>(d / 32);
  const dim3 grid(static_cast<unsigned>(P * (f / (2 * kMxRows))));
#define MOE_BMX_GUS(CI_, S_)                                                                                     \
  hipLaunchKernelGGL((batched_mx_gateup_kernel<CI_, S_>), grid, dim3(256), 0, as_stream(stream),                 \
                     static_cast<const uint16_t*>(x), topk_ids, logits, static_cast<int>(score), topk_w,          \
                     static_cast<const uint8_t*>(wq_gate_up), static_cast<const uint8_t*>(ws_gate_up),           \
                     static_cast<int>(P), k, E, static_cast<int>(d), static_cast<int>(f), static_cast<uint16_t*>(h))
#define MOE_BMX_GUS_CI(S_)            \
  if (KB <= 64) MOE_BMX_GUS(1, S_);   \
  else if (KB <= 128) MOE_BMX_GUS(2, S_); \
  else MOE_BMX_GUS(4, S_)
  if (E <= 64) {
    MOE_BMX_GUS_CI(1);
  } else if (E <= 128) {
    MOE_BMX_GUS_CI(2);
  } else {
    MOE_BMX_GUS_CI(4);
  }
#undef MOE_BMX_GUS_CI
#undef MOE_BMX_GUS
  return launch_status();
}

extern "C" moe_status moe_batched_down_combine_mxfp4(const void* h, const int32_t* topk_ids, const float* topk_w,
                                                     const void* wq_down, const void* ws_down, const void* y_shared,
                                                     int64_t T, int64_t d, int64_t f, int32_t E, int32_t k, void* y,
                                                     void* stream) {
  moe_status s = check_batched_mx(h, topk_ids, wq_down, ws_down, T, d, f, E, k, y);
  if (s != MOE_OK || T == 0) return s;
  if (!topk_w) return MOE_ERR_INVALID_ARG;
  const int KB = static_cast<int>(f / 32);
  const dim3 grid(static_cast<unsigned>(T * (d / kMxRows)));
#define MOE_BMX_DN(CI_)                                                                                          \
  hipLaunchKernelGGL((batched_mx_down_combine_kernel<CI_>), grid, dim3(256), 0, as_stream(stream),              \
                     static_cast<const uint16_t*>(h), topk_ids, topk_w, static_cast<const uint8_t*>(wq_down),     \
                     static_cast<const uint8_t*>(ws_down), static_cast<const uint16_t*>(y_shared),                \
                     static_cast<int>(T), k, E, static_cast<int>(f), static_cast<int>(d), static_cast<uint16_t*>(y))
  if (KB <= 64) MOE_BMX_DN(1);
  else if (KB <= 128) MOE_BMX_DN(2);
  else MOE_BMX_DN(4);
#undef MOE_BMX_DN
  return launch_status();
}

extern "C" moe_status moe_decode_gateup_swiglu_mxfp4(const void* x, const int32_t* perm, int32_t k,
                                                     const void* wq_gate_up, const void* ws_gate_up,
                                                     const int32_t* offsets, int64_t rows, int64_t d, int64_t f,
                                                     int32_t E, void* h, void* stream) {
  moe_status s = check_mx(x, wq_gate_up, ws_gate_up, offsets, rows, d, f, E, h, d);
  if (s != MOE_OK || rows == 0) return s;
  if (perm && (k < 1 || k > kMaxK || rows % k != 0)) return MOE_ERR_INVALID_ARG;
  if (rows > kMxVectorRowsPerExpert * E)
    return launch_mx_mfma<true>(x, wq_gate_up, ws_gate_up, offsets, perm, perm ? k : 1, rows, d, f, E, h,
                                as_stream(stream));
  return launch_mx<true>(x, wq_gate_up, ws_gate_up, offsets, perm, perm ? k : 1, rows, d, f, E, h, as_stream(stream));
}

extern "C" moe_status moe_decode_down_mxfp4(const void* h, const void* wq_down, const void* ws_down,
                                            const int32_t* offsets, int64_t rows, int64_t d, int64_t f, int32_t E,
                                            void* y_perm, void* stream) {
  moe_status s = check_mx(h, wq_down, ws_down, offsets, rows, d, f, E, y_perm, f);
  if (s != MOE_OK || rows == 0) return s;
  if (rows > kMxVectorRowsPerExpert * E)
    return launch_mx_mfma<false>(h, wq_down, ws_down, offsets, nullptr, 1, rows, f, d, E, y_perm, as_stream(stream));
  return launch_mx<false>(h, wq_down, ws_down, offsets, nullptr, 1, rows, f, d, E, y_perm, as_stream(stream));
}
