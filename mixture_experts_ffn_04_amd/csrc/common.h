// Shared device helpers and host-side argument checks for libmoe (gfx950).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "libmoe.h"

namespace moe {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

constexpr int kWave = 64;
constexpr int kMaxE = 256;
constexpr int kMaxK = 16;

// ---------------------------------------------------------------- bf16

__device__ __forceinline__ float bf16_to_f32(uint16_t b) {
  return __uint_as_float(static_cast<uint32_t>(b) << 16);
}

// Round to nearest even (hardware v_cvt_pk_bf16_f32 on gfx950).
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  return __builtin_bit_cast(uint16_t, static_cast<__bf16>(f));
}

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return static_cast<uint32_t>(f32_to_bf16(lo)) | (static_cast<uint32_t>(f32_to_bf16(hi)) << 16);
}

// silu(g) = g * sigmoid(g), with the hardware reciprocal (v_rcp_f32, about
// 1 ulp) in place of an IEEE division: the SwiGLU output is rounded to bf16
// right after, and the division's scale/fixup sequence made the gate/up
// epilogue VALU-bound (measured: c4 gate/up 458 -> 449 us).
__device__ __forceinline__ float silu(float g) { return g * __builtin_amdgcn_rcpf(1.0f + __expf(-g)); }

typedef __bf16 bfx2 __attribute__((ext_vector_type(2)));

// acc + w.x (two bf16 pairs, fp32 accumulate: v_dot2_f32_bf16)
__device__ __forceinline__ float dot2(unsigned w, unsigned x, float acc) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bfx2, w), __builtin_bit_cast(bfx2, x), acc, false);
}

// acc + w.x over 16 bytes (8 bf16) of each
__device__ __forceinline__ float dot8(const u32x4& w, const u32x4& x, float acc) {
  acc = dot2(w.x, x.x, acc);
  acc = dot2(w.y, x.y, acc);
  acc = dot2(w.z, x.z, acc);
  return dot2(w.w, x.w, acc);
}

// ---------------------------------------------------------------- waves

__device__ __forceinline__ int lane_id() { return __lane_id(); }

// Clamp an offsets entry read from device memory to [0, rows].
__host__ __device__ __forceinline__ int clamp_off(int v, int rows) { return v < 0 ? 0 : (v > rows ? rows : v); }

// Index of the j-th group with rows (in group order), or -1; all 256
// threads of the workgroup call it (G <= 256).  A decode batch of P < G
// rows touches at most P groups, so the grid then covers only P groups and
// no workgroup is spent on an expert without tokens (with P >= G the grid
// covers every group and empty ones exit at once, which measured faster
// than the search).
__device__ __forceinline__ int nth_active_group(const int32_t* __restrict__ off, int G, int rows, int j) {
  __shared__ int s_cnt[4];
  __shared__ int s_g;
  const int t = threadIdx.x, lane = t & 63, w = t >> 6;
  bool act = false;
  if (t < G) act = clamp_off(off[t + 1], rows) > clamp_off(off[t], rows);
  const uint64_t m = __ballot(act);
  if (lane == 0) s_cnt[w] = __popcll(m);
  if (t == 0) s_g = -1;
  __syncthreads();
  int rank = __popcll(m & ((uint64_t(1) << lane) - 1));
  for (int i = 0; i < w; ++i) rank += s_cnt[i];
  if (act && rank == j) s_g = t;
  __syncthreads();
  return s_g;
}

// MXFP4 (OCP Microscaling): E8M0 scale code -> 2^(code - 127) as fp32
// (code 0: 2^-127, a denormal; code 255: NaN), with selects rather than
// branches, so no load waits on the decode of an earlier one.
__device__ __forceinline__ float e8m0_to_f32(uint32_t code) {
  uint32_t b = code << 23;
  b = code == 0u ? 0x00400000u : b;
  b = code == 255u ? 0x7fc00000u : b;
  return __uint_as_float(b);
}

// ---------------------------------------------------------------- host

inline bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

inline int elem_bytes(moe_dtype dt) { return dt == MOE_BF16 ? 2 : 4; }

inline bool valid_dtype(moe_dtype dt) { return dt == MOE_BF16 || dt == MOE_F32; }

inline moe_status launch_status() {
  hipError_t e = hipGetLastError();
  return e == hipSuccess ? MOE_OK : MOE_ERR_HIP;
}

inline hipStream_t as_stream(void* s) { return reinterpret_cast<hipStream_t>(s); }

inline int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

}  // namespace moe
