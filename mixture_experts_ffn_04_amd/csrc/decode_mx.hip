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
// Two forms, by rows per expert.  From one row per expert on average, the
// LDS-staged MFMA form (decode_mx_lds_kernel, below).  With fewer rows, the
// vector form: workgroup = (expert g with rows, CPB output columns), 4
// waves; each wave owns R = 4 weight rows (gate/up: the gate and up rows of
// 2 columns; down: 4 columns).  Lane l keeps blocks l, l + 64, ... of its
// 4 rows in registers (16 code bytes and one scale per block), loaded once:
// the expert's weights are read from HBM once.  Then for every token row of the
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
// From this many rows per expert on average the LDS-staged MFMA form runs
// (measured faster from one row per expert of the 32-expert workload); the
// vector form re-reads each activation row for every 4 weight rows.
constexpr int64_t kMxStagedRowsPerExpert = 1;

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
// writes the token's ids and weights.  The token's activation row is read
// once per workgroup into LDS (its loads issued first, written to LDS after
// the weight loads are issued), so a lane holds only its weight blocks while
// their loads are in flight: the 5760 waves of one token with four experts
// of the gpt-oss shape then make one round instead of 1.1 at the five waves
// per SIMD that register-held activations allowed.  A row of K <= 2048 CI
// elements is 256 CI chunks of 16 bytes: CI per thread.

template <int CI>
__device__ __forceinline__ void mx_dot_rows_lds(const u32x4 (&wq)[kMxRows][CI], const uint32_t (&ws)[kMxRows][CI],
                                                const u32x4* xs, int KB, int lane, float (&acc)[kMxRows]) {
#pragma unroll
  for (int r = 0; r < kMxRows; ++r) acc[r] = 0.0f;
#pragma unroll
  for (int i = 0; i < CI; ++i) {
    const int b = lane + 64 * i;
    if (b < KB) {
      u32x4 xv[4];
#pragma unroll
      for (int c = 0; c < 4; ++c) xv[c] = xs[b * 4 + c];
#pragma unroll
      for (int r = 0; r < kMxRows; ++r) acc[r] = fmaf(block_dot(wq[r][i], xv), e8m0_to_f32(ws[r][i]), acc[r]);
    }
  }
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) {
#pragma unroll
    for (int r = 0; r < kMxRows; ++r) acc[r] += __shfl_xor(acc[r], o, 64);
  }
}

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
  if (p >= P) return;                                    // uniform over the workgroup
  // the token's row: K / 8 chunks of 16 bytes, at most CI per thread
  const uint16_t* xr = x + static_cast<int64_t>(p / k) * K;
  const int nx = K / 8;
  u32x4 xc[CI];
#pragma unroll
  for (int i = 0; i < CI; ++i) {
    const int c = threadIdx.x + 256 * i;
    if (c < nx) xc[i] = *(const gu4*)(xr + c * 8);
  }
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
  if (e < 0 || e >= E) return;                           // a pair of an expert held elsewhere (uniform)
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int n0 = cb * CPB + wave * CPW;
  const int KB = K / 32;
  int wr[kMxRows];
  mx_wave_rows<true>(n0, N, wr);
  u32x4 wq[kMxRows][CI];
  uint32_t ws[kMxRows][CI];
  mx_load_rows<CI>(Bq + static_cast<int64_t>(e) * 2 * N * (K / 2), Bs + static_cast<int64_t>(e) * 2 * N * KB, wr, K,
                   KB, lane, wq, ws);
  __shared__ u32x4 xs[256 * CI];
#pragma unroll
  for (int i = 0; i < CI; ++i) {
    const int c = threadIdx.x + 256 * i;
    if (c < nx) xs[c] = xc[i];
  }
  __syncthreads();
  float acc[kMxRows];
  mx_dot_rows_lds<CI>(wq, ws, xs, KB, lane, acc);
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
// Several rows per expert: one MX quad (4 blocks, 128 elements of K) of a
// 16-row weight tile against 16 token rows on v_mfma_f32_16x16x32_bf16,
// weight rows as the 16-row operand and tokens as the 16-column one.  Lane
// (i = lane % 16, q = lane / 16) holds block q of weight row i (16 code
// bytes and one scale code) and the 32 elements of token i under it; MFMA m
// takes elements 8m .. 8m + 7 of every lane's block, of the weights and the
// tokens alike, which only permutes the order of the reduction over K.  The
// gfx950 FP4 conversion applies the block's power of two while decoding, so
// the bf16 operand is the weight's value.
struct MxQuad {
  u32x4 c;       // codes of block q of weight row i
  uint32_t s;    // its scale code (raw)
  u32x4 t[4];    // t[m]: elements 8m .. 8m + 7 of the block, of token i
};

// The quad's 4 MFMAs into acc.
__device__ __forceinline__ void mx_quad_mma(const MxQuad& s, f32x4& acc) {
  typedef bf16x2v b2;
  const float f = e8m0_to_f32(s.s);
#pragma unroll
  for (int m = 0; m < 4; ++m) {
    u32x4 w;
    w[0] = __builtin_bit_cast(uint32_t, (b2)__builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(s.c[m], f, 0));
    w[1] = __builtin_bit_cast(uint32_t, (b2)__builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(s.c[m], f, 1));
    w[2] = __builtin_bit_cast(uint32_t, (b2)__builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(s.c[m], f, 2));
    w[3] = __builtin_bit_cast(uint32_t, (b2)__builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(s.c[m], f, 3));
    acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, w), __builtin_bit_cast(bf16x8, s.t[m]),
                                                  acc, 0, 0, 0);
  }
}

// ---------------------------------------------------------------------------
// Several rows per expert, LDS-staged form.  Workgroup = (expert g, 64
// weight rows): gate/up the gate and up rows of 32 output columns, down 64
// output columns.  Wave w owns one 16-row tile of them and one chunk of up
// to 16 of the expert's token rows: gate/up rows 0-7 of the tile are the
// gate rows and rows 8-15 the up rows of columns 8w .. 8w + 7, down the
// rows of columns 16w .. 16w + 15.  Every operand reaches LDS by
// direct-to-LDS loads of 1 KB contiguous in LDS: first the scales of the
// 64 rows for the whole of K (contiguous pieces of the scale tensor), then
// stages of two quads (256 elements of K): 128 bytes of codes of each weight
// row (8 rows per load) and 512 bytes of each token row (2 rows per load,
// gathered through the row map), in a ring of stage buffers (4 in the wide
// LDS shape, three stages in flight while one is used; 2 in the others, see
// MxlShape).  Whole 128-byte row pieces per load measured faster than
// 64-byte ones (c3mx T=64 gate/up 62.7 against 66.7 us); 80 KB of LDS lets
// two workgroups share a CU (48 KB: three, 40 KB: four), so one's first
// loads and last stores hide under another's stream.  Chunk c of a 128-byte
// code row r sits at c ^ ((r / 2) % 8) and chunk c of a 512-byte token row
// r at c ^ (r % 16), so the 16 rows a wave reads at one chunk hit distinct
// banks.  The MFMAs take the layout of MxQuad.  Loads past a buffer's end
// read zeros (buffer range check); the elements of a last stage past K are
// read but never used (loading only the pieces inside K measured 1-2%
// slower).
typedef __attribute__((address_space(3))) void mxl_lds_void;

constexpr int kMxlRows = 64;                                   // weight rows per workgroup
constexpr int kMxlCodeBytes = kMxlRows * 128;                  // per stage: 128 bytes of each row
constexpr int kMxlTokBytes = 16 * 512;                         // per stage: 512 bytes of 16 token rows
constexpr int kMxlStageBytes = kMxlCodeBytes + kMxlTokBytes;
// LDS shapes: NS stage buffers and a scale area of SCB bytes (the 64 rows'
// K / 32 scale bytes each, so K <= SCB / 2).  Gate/up takes the narrow one
// for K <= 4096 (2 stages, 40 KB: four workgroups per CU), the wide one
// above (4 stages, K <= 8192, 80 KB: two per CU); down takes the middle one
// (2 stages, K <= 8192, 48 KB: three per CU).  A shape with fewer stages
// keeps fewer bytes in flight per workgroup, but the CU holds more
// workgroups, whose phases drift apart, and the launch's rounds change.
// Same-box A/B, c3mx at T=32 / T=64: gate/up narrow against wide 65 -> 61 /
// 68 -> 66 us; down narrow against wide 37 -> 40 us at T=64 (1,440
// workgroups of 64 columns at d = 2880 make 1.4 rounds of four per CU),
// middle against wide 35.2 -> 33.4 / 36.9 -> 35.9 us (steps -2%).
template <int NS, int SCB>
struct MxlShape {
  static constexpr int kStages = NS;
  static constexpr int kScaleBytes = SCB;
  static constexpr int kLdsBytes = SCB + NS * kMxlStageBytes;
  static constexpr int kPerCu = (160 * 1024) / kLdsBytes;
};
typedef MxlShape<4, kMxlRows * 256> MxlWide;
typedef MxlShape<2, kMxlRows * 128> MxlNarrow;
typedef MxlShape<2, kMxlRows * 256> MxlMid;
static_assert(MxlWide::kPerCu == 2 && MxlMid::kPerCu == 3 && MxlNarrow::kPerCu == 4, "workgroups per CU");
constexpr int kMxlOob = 0x7fff0000;                            // a lane offset past every buffer
constexpr int kMxlBufFlags = 0x00020000;                       // raw untyped 32-bit accesses (gfx9)

// One LDS DMA: 64 lanes x 16 bytes from buffer rs at lane offset voff into
// LDS [lds_addr, lds_addr + 1024).  Asm, so the compiler adds no wait of its
// own for it; the kernel waits with vmcnt before the barrier that publishes
// a stage.  No register outputs; nothing else here uses m0.
__device__ __forceinline__ void mxl_dma16(__amdgpu_buffer_rsrc_t rs, int voff, unsigned lds_addr) {
  asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tbuffer_load_dwordx4 %0, %1, 0 offen lds"
               :: "v"(voff), "s"(rs), "s"(lds_addr) : "memory", "m0");
}

// This wave's loads but the VM youngest have landed and its LDS reads are
// done, then the barrier: every wave's loads of the stage are visible and
// the buffer read before is free.
template <int VM>
__device__ __forceinline__ void mxl_wait_barrier() {
  static_assert(VM < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((VM & 15) | (7 << 4) | (0 << 8) | ((VM >> 4) << 14));
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// The form's address arithmetic, shared by the kernel and by the host
// replay that checks it (tests/mx_lds_replay.cpp), so __host__ __device__.
//
// Expert row of local weight row r (0 .. 63) of the block at output column
// n0: gate/up tile t = r / 16 holds gate rows n0 + 8t .. and up rows
// N + n0 + 8t ..; down rows are n0 + r.
template <bool SWIGLU>
__host__ __device__ __forceinline__ int mxl_expert_row(int r, int n0, int N) {
  if (!SWIGLU) return n0 + r;
  const int t = r >> 4, h = r & 15;
  return h < 8 ? n0 + 8 * t + h : N + n0 + 8 * t + h - 8;
}

// LDS scale row of local weight row r: gate/up [gate rows n0 .. n0 + 31][up
// rows N + n0 .. N + n0 + 31], down rows n0 .. n0 + 63.
template <bool SWIGLU>
__host__ __device__ __forceinline__ int mxl_scale_row(int r) {
  if (!SWIGLU) return r;
  const int t = r >> 4, h = r & 15;
  return h < 8 ? 8 * t + h : 32 + 8 * t + h - 8;
}

// Scales as [64][KB] bytes in LDS: byte offset in the expert's scales of
// 16-byte chunk c (gate rows n0 .. for c < 2 KB, up rows N + n0 .. after;
// down rows n0 ..), or kMxlOob past the 64 rows.
template <bool SWIGLU>
__host__ __device__ __forceinline__ int mxl_scale_off(int c, int n0, int N, int KB) {
  if (c >= 4 * KB) return kMxlOob;
  const int b = 16 * c;
  return (SWIGLU && b >= 32 * KB) ? (N + n0) * KB + b - 32 * KB : n0 * KB + b;
}

// Code load kk (0, 1) of wave w fills local rows 8 (2w + kk) .. + 7, 128
// bytes each: the lane's local row, and its byte offset in the expert's
// codes at stage 0 (stage st adds 128 st).  Chunk c of row r goes to slot
// c ^ ((r / 2) % 8) of the row in LDS.
__host__ __device__ __forceinline__ int mxl_code_row(int wave, int kk, int lane) {
  return 16 * wave + 8 * kk + (lane >> 3);
}

template <bool SWIGLU>
__host__ __device__ __forceinline__ int mxl_code_off(int wave, int kk, int lane, int n0, int N, int KH) {
  const int r = mxl_code_row(wave, kk, lane);
  const int chunk = (lane & 7) ^ ((r >> 1) & 7);
  return mxl_expert_row<SWIGLU>(r, n0, N) * KH + chunk * 16;
}

// Token load kk of wave w fills token rows 4w + 2kk and 4w + 2kk + 1 of the
// chunk, 512 bytes each: the lane's row, and its byte offset in A at stage
// 0 for source row src (stage st adds 512 st), or kMxlOob without one.
// Chunk c of row r goes to slot c ^ (r % 16).
__host__ __device__ __forceinline__ int mxl_tok_row(int wave, int kk, int lane) {
  return 4 * wave + 2 * kk + (lane >> 5);
}

__host__ __device__ __forceinline__ int mxl_tok_off(int src, int K, int wave, int kk, int lane) {
  const int tr = mxl_tok_row(wave, kk, lane);
  return src >= 0 ? src * (K * 2) + (((lane & 31) ^ (tr & 15)) * 16) : kMxlOob;
}

// Token loads a wave issues per stage for a chunk of `left` rows (those
// whose two rows both lie past the chunk are skipped).
__host__ __device__ __forceinline__ int mxl_tok_loads(int left, int wave) {
  const int n = (left - 4 * wave + 1) / 2;
  return n < 0 ? 0 : (n > 2 ? 2 : n);
}

// LDS offsets a lane reads in quad u of a stage buffer: the codes of block
// 4u + q of local row rl, and elements 8m .. 8m + 7 of that block of token
// row i (from the buffer's code and token parts).
__host__ __device__ __forceinline__ int mxl_code_read(int rl, int u, int q) {
  return rl * 128 + (((4 * u + q) ^ ((rl >> 1) & 7)) * 16);
}

__host__ __device__ __forceinline__ int mxl_tok_read(int i, int u, int q, int m) {
  return i * 512 + (((16 * u + 4 * q + m) ^ i) * 16);
}

// rows >= G: every group has workgroups (those of groups without rows exit).
// SH: the LDS shape (MxlWide or MxlNarrow).
template <bool SWIGLU, typename SH>
__global__ __launch_bounds__(256, SH::kPerCu) void decode_mx_lds_kernel(const uint16_t* __restrict__ A,
                                                               const uint8_t* __restrict__ Bq,
                                                               const uint8_t* __restrict__ Bs,
                                                               const int32_t* __restrict__ off,
                                                               const int32_t* __restrict__ rowmap, int kdiv,
                                                               int rows, int K, int N, uint16_t* __restrict__ C) {
  constexpr int NS = SH::kStages, SCB = SH::kScaleBytes;
  __shared__ __attribute__((aligned(1024))) uint8_t lds[SH::kLdsBytes];
  constexpr int CPB = SWIGLU ? 32 : 64;                 // output columns per workgroup
  const int ncb = (N + CPB - 1) / CPB;
  const int g = blockIdx.x / ncb;
  const int cb = blockIdx.x - g * ncb;
  const int lo = clamp_off(off[g], rows);
  const int hi = clamp_off(off[g + 1], rows);
  if (hi <= lo) return;                                 // expert without rows: its weights are never read
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x) >> 6);
  const int i16 = lane & 15, part = lane >> 4;
  const int n0 = cb * CPB;
  const int KB = K / 32, KH = K / 2;
  const int nq = KB / 4;                                // whole quads; K % 128 == 64 adds a half quad
  const int nst = (K + 255) / 256;
  const int brows = SWIGLU ? 2 * N : N;
  const unsigned lds0 = static_cast<unsigned>(reinterpret_cast<uintptr_t>((const mxl_lds_void*)lds));
  const __amdgpu_buffer_rsrc_t crs = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint8_t*>(Bq) + static_cast<int64_t>(g) * brows * KH, 0, brows * KH, kMxlBufFlags);
  const __amdgpu_buffer_rsrc_t srs = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint8_t*>(Bs) + static_cast<int64_t>(g) * brows * KB, 0, brows * KB, kMxlBufFlags);
  const __amdgpu_buffer_rsrc_t trs = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint16_t*>(A), 0, (rows / kdiv) * K * 2, kMxlBufFlags);

  // The 64 rows' scales for the whole of K, [64][KB] bytes.
  for (int k = wave; k * 64 < 4 * KB; k += 4)
    mxl_dma16(srs, mxl_scale_off<SWIGLU>(k * 64 + lane, n0, N, KB), __builtin_amdgcn_readfirstlane(lds0 + k * 1024));

  // Code loads: wave w fills local rows 16 w .. 16 w + 15, 8 per load.
  int cvo[2];
#pragma unroll
  for (int kk = 0; kk < 2; ++kk) cvo[kk] = mxl_code_off<SWIGLU>(wave, kk, lane, n0, N, KH);
  // The lane's weight row (row i16 of the wave's tile).
  const int rl = 16 * wave + i16;
  const int sl = mxl_scale_row<SWIGLU>(rl) * KB;

  for (int m0 = lo; m0 < hi; m0 += 16) {
    // Token loads: wave w fills token rows 4 w .. 4 w + 3, 2 per load; the
    // rows' sources are wave-uniform (scalar loads).
    int tvo[2];
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
      int src[2];
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int m = m0 + 4 * wave + 2 * kk + h;
        int sr = -1;
        if (m < hi) sr = rowmap ? clamp_off(rowmap[m], rows - 1) / kdiv : m;
        src[h] = __builtin_amdgcn_readfirstlane(sr);
      }
      tvo[kk] = mxl_tok_off((lane >> 5) ? src[1] : src[0], K, wave, kk, lane);
    }
    // A token load whose two rows both lie past the expert's rows is not
    // issued: the wave issues 2 + ntl loads per stage.  Those rows' LDS
    // keeps older data, which only reaches the MFMA columns of token rows
    // that are never stored.
    const int ntl = mxl_tok_loads(hi - m0, wave);
    auto dma_stage = [&](int st, int buf) {
      const unsigned sb = lds0 + SCB + buf * kMxlStageBytes;
#pragma unroll
      for (int kk = 0; kk < 2; ++kk)
        mxl_dma16(crs, cvo[kk] + st * 128, __builtin_amdgcn_readfirstlane(sb + (2 * wave + kk) * 1024));
#pragma unroll
      for (int kk = 0; kk < 2; ++kk)
        if (kk < ntl)
          mxl_dma16(trs, tvo[kk] + st * 512,
                    __builtin_amdgcn_readfirstlane(sb + kMxlCodeBytes + (2 * wave + kk) * 1024));
    };
    for (int st = 0; st < NS - 1 && st < nst; ++st) dma_stage(st, st);
    f32x4 acc = {};
    for (int st = 0; st < nst; ++st) {
      // this wave's later stages in flight: (ahead) x (2 + ntl) loads
      switch (min(nst - 1 - st, NS - 2) * (2 + ntl)) {
        case 8: mxl_wait_barrier<8>(); break;
        case 6: mxl_wait_barrier<6>(); break;
        case 4: mxl_wait_barrier<4>(); break;
        case 3: mxl_wait_barrier<3>(); break;
        case 2: mxl_wait_barrier<2>(); break;
        default: mxl_wait_barrier<0>(); break;
      }
      if (st + NS - 1 < nst) dma_stage(st + NS - 1, (st + NS - 1) % NS);
      const uint8_t* cbuf = lds + SCB + (st % NS) * kMxlStageBytes;
      const uint8_t* tbuf = cbuf + kMxlCodeBytes;
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        const int jq = 2 * st + u;                      // the quad
        if (jq > nq || (jq == nq && !(KB & 3))) break;  // past K
        MxQuad t;
        t.c = *reinterpret_cast<const u32x4*>(cbuf + mxl_code_read(rl, u, part));
        t.s = lds[sl + 4 * jq + part];
#pragma unroll
        for (int m = 0; m < 4; ++m) t.t[m] = *reinterpret_cast<const u32x4*>(tbuf + mxl_tok_read(i16, u, part, m));
        if (jq == nq && part >= 2) {                    // K % 128 == 64: blocks 2 and 3 of the last quad are past K
          const u32x4 zero = {0u, 0u, 0u, 0u};
          t.c = zero;
          t.s = 127u;
#pragma unroll
          for (int m = 0; m < 4; ++m) t.t[m] = zero;
        }
        mx_quad_mma(t, acc);
      }
    }
    // lane (token i16, part) holds tile rows 4 part .. 4 part + 3
    const int row = m0 + i16;
    uint2 v;
    if (SWIGLU) {
      // gate rows (parts 0, 1) meet their up rows (parts 2, 3) 32 lanes up
      float up[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const unsigned gb = __float_as_uint(acc[r]);
        up[r] = __uint_as_float(__builtin_amdgcn_permlane32_swap(gb, gb, false, false)[1]);
      }
      if (part < 2 && row < hi && n0 + 8 * wave < N) {
        v.x = pack_bf16x2(silu(acc[0]) * up[0], silu(acc[1]) * up[1]);
        v.y = pack_bf16x2(silu(acc[2]) * up[2], silu(acc[3]) * up[3]);
        *reinterpret_cast<uint2*>(C + static_cast<int64_t>(row) * N + n0 + 8 * wave + 4 * part) = v;
      }
    } else if (row < hi && n0 + 16 * wave < N) {
      v.x = pack_bf16x2(acc[0], acc[1]);
      v.y = pack_bf16x2(acc[2], acc[3]);
      *reinterpret_cast<uint2*>(C + static_cast<int64_t>(row) * N + n0 + 16 * wave + 4 * part) = v;
    }
    __syncthreads();                                    // every wave is done with the buffers the next chunk loads
  }
}

template <bool SWIGLU>
moe_status launch_mx_lds(const void* A, const void* Bq, const void* Bs, const int32_t* off, const int32_t* rowmap,
                         int kdiv, int64_t rows, int64_t K, int64_t N, int G, void* C, hipStream_t st) {
  constexpr int CPB = SWIGLU ? 32 : 64;
  if (rows < G) return MOE_ERR_UNSUPPORTED;               // the callers take the vector form then
  const int64_t grid = static_cast<int64_t>(G) * ((N + CPB - 1) / CPB);
  if (grid > 0x7fffffff) return MOE_ERR_UNSUPPORTED;
#define MOE_MXL_LAUNCH(SH_)                                                                                   \
  hipLaunchKernelGGL((decode_mx_lds_kernel<SWIGLU, SH_>), dim3(static_cast<unsigned>(grid)), dim3(256), 0, st,    \
                     static_cast<const uint16_t*>(A), static_cast<const uint8_t*>(Bq),                         \
                     static_cast<const uint8_t*>(Bs), off, rowmap, kdiv, static_cast<int>(rows),               \
                     static_cast<int>(K), static_cast<int>(N), static_cast<uint16_t*>(C))
  if constexpr (SWIGLU) {
    if (K <= MxlNarrow::kScaleBytes / 2) MOE_MXL_LAUNCH(MxlNarrow);
    else MOE_MXL_LAUNCH(MxlWide);
  } else {
    MOE_MXL_LAUNCH(MxlMid);
  }
#undef MOE_MXL_LAUNCH
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
  // K bounds the scale rows the LDS-staged form keeps; d * f bounds one
  // expert's codes (d f bytes for gate/up) so 32-bit buffer offsets reach them
  if (E > kMaxE || rows > kMxMaxRows || K > MxlWide::kScaleBytes / 2 || d * f > (int64_t(1) << 30))
    return MOE_ERR_UNSUPPORTED;
  if (d % 64 != 0 || f % 64 != 0) return MOE_ERR_ALIGNMENT;
  if (rows == 0) return MOE_OK;
  if (!in || !wq || !ws || !offsets || !out) return MOE_ERR_INVALID_ARG;
  if (!aligned16(in) || !aligned16(wq) || !aligned16(ws) || !aligned16(out)) return MOE_ERR_ALIGNMENT;
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
  if (rows >= kMxStagedRowsPerExpert * E)
    return launch_mx_lds<true>(x, wq_gate_up, ws_gate_up, offsets, perm, perm ? k : 1, rows, d, f, E, h,
                                as_stream(stream));
  return launch_mx<true>(x, wq_gate_up, ws_gate_up, offsets, perm, perm ? k : 1, rows, d, f, E, h, as_stream(stream));
}

extern "C" moe_status moe_decode_down_mxfp4(const void* h, const void* wq_down, const void* ws_down,
                                            const int32_t* offsets, int64_t rows, int64_t d, int64_t f, int32_t E,
                                            void* y_perm, void* stream) {
  moe_status s = check_mx(h, wq_down, ws_down, offsets, rows, d, f, E, y_perm, f);
  if (s != MOE_OK || rows == 0) return s;
  if (rows >= kMxStagedRowsPerExpert * E)
    return launch_mx_lds<false>(h, wq_down, ws_down, offsets, nullptr, 1, rows, f, d, E, y_perm, as_stream(stream));
  return launch_mx<false>(h, wq_down, ws_down, offsets, nullptr, 1, rows, f, d, E, y_perm, as_stream(stream));
}
