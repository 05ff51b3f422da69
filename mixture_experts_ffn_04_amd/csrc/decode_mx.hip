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

namespace moe {
namespace {

typedef __attribute__((address_space(1))) const u32x4 gu4;
typedef __bf16 bf16x2v __attribute__((ext_vector_type(2)));

constexpr int kMxRows = 4;            // weight rows per wave
constexpr int64_t kMxMaxRows = 1024;  // routed rows per call (decode sizes)

// E8M0 scale code -> 2^(code - 127) as fp32 (code 0: 2^-127, a denormal;
// code 255: NaN).
__device__ __forceinline__ float e8m0_to_f32(uint32_t code) {
  if (code == 0) return __uint_as_float(0x00400000u);
  if (code == 255) return __uint_as_float(0x7fc00000u);
  return __uint_as_float(code << 23);
}

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
  const uint8_t* Bqg = Bq + static_cast<int64_t>(g) * brows * (K / 2);
  const uint8_t* Bsg = Bs + static_cast<int64_t>(g) * brows * KB;
  int wr[kMxRows];
#pragma unroll
  for (int r = 0; r < kMxRows; ++r) wr[r] = SWIGLU ? (r < 2 ? n0 + r : N + n0 + r - 2) : n0 + r;
  const u32x4 zero = {0u, 0u, 0u, 0u};
  u32x4 wq[kMxRows][CI];
  float ws[kMxRows][CI];
#pragma unroll
  for (int r = 0; r < kMxRows; ++r) {
#pragma unroll
    for (int i = 0; i < CI; ++i) {
      const int b = lane + 64 * i;
      const bool ok = b < KB;
      wq[r][i] = ok ? *(const gu4*)(Bqg + static_cast<int64_t>(wr[r]) * (K / 2) + b * 16) : zero;
      ws[r][i] = ok ? e8m0_to_f32(Bsg[static_cast<int64_t>(wr[r]) * KB + b]) : 0.0f;
    }
  }
  for (int m = lo; m < hi; ++m) {
    const int src = rowmap ? clamp_off(rowmap[m], rows - 1) / kdiv : m;
    const uint16_t* xr = A + static_cast<int64_t>(src) * K;
    float acc[kMxRows] = {};
#pragma unroll
    for (int i = 0; i < CI; ++i) {
      const int b = lane + 64 * i;
      if (b < KB) {
        u32x4 xv[4];
#pragma unroll
        for (int c = 0; c < 4; ++c) xv[c] = *(const gu4*)(xr + b * 32 + c * 8);
#pragma unroll
        for (int r = 0; r < kMxRows; ++r) acc[r] = fmaf(block_dot(wq[r][i], xv), ws[r][i], acc[r]);
      }
    }
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) {
#pragma unroll
      for (int r = 0; r < kMxRows; ++r) acc[r] += __shfl_xor(acc[r], o, 64);
    }
    if (lane == 0) {
      uint16_t* crow = C + static_cast<int64_t>(m) * N + n0;
      if (SWIGLU) {
        *reinterpret_cast<uint32_t*>(crow) = pack_bf16x2(silu(acc[0]) * acc[2], silu(acc[1]) * acc[3]);
      } else {
        uint2 v;
        v.x = pack_bf16x2(acc[0], acc[1]);
        v.y = pack_bf16x2(acc[2], acc[3]);
        *reinterpret_cast<uint2*>(crow) = v;
      }
    }
  }
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

}  // namespace
}  // namespace moe

using namespace moe;

extern "C" moe_status moe_decode_gateup_swiglu_mxfp4(const void* x, const int32_t* perm, int32_t k,
                                                     const void* wq_gate_up, const void* ws_gate_up,
                                                     const int32_t* offsets, int64_t rows, int64_t d, int64_t f,
                                                     int32_t E, void* h, void* stream) {
  moe_status s = check_mx(x, wq_gate_up, ws_gate_up, offsets, rows, d, f, E, h, d);
  if (s != MOE_OK || rows == 0) return s;
  if (perm && (k < 1 || k > kMaxK || rows % k != 0)) return MOE_ERR_INVALID_ARG;
  return launch_mx<true>(x, wq_gate_up, ws_gate_up, offsets, perm, perm ? k : 1, rows, d, f, E, h, as_stream(stream));
}

extern "C" moe_status moe_decode_down_mxfp4(const void* h, const void* wq_down, const void* ws_down,
                                            const int32_t* offsets, int64_t rows, int64_t d, int64_t f, int32_t E,
                                            void* y_perm, void* stream) {
  moe_status s = check_mx(h, wq_down, ws_down, offsets, rows, d, f, E, y_perm, f);
  if (s != MOE_OK || rows == 0) return s;
  return launch_mx<false>(h, wq_down, ws_down, offsets, nullptr, 1, rows, f, d, E, y_perm, as_stream(stream));
}
