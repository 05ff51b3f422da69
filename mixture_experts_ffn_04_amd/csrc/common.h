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

__device__ __forceinline__ float silu(float g) { return g / (1.0f + __expf(-g)); }

// ---------------------------------------------------------------- waves

__device__ __forceinline__ int lane_id() { return __lane_id(); }

// Clamp an offsets entry read from device memory to [0, rows].
__device__ __forceinline__ int clamp_off(int v, int rows) { return v < 0 ? 0 : (v > rows ? rows : v); }

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
