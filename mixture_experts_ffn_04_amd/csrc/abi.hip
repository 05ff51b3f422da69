// C ABI entry points for the expert projections, plus version / status
// helpers.  Argument checks run on the host before any launch.
#include "grouped_gemm.h"

namespace moe {
moe_status gemm_bf16_gateup_swiglu(const GemmArgs& a, hipStream_t st);
moe_status gemm_bf16_down(const GemmArgs& a, hipStream_t st);
moe_status gemm_bf16_gateup_swiglu_few(const GemmArgs& a, hipStream_t st);
moe_status gemm_bf16_down_few(const GemmArgs& a, hipStream_t st);
moe_status gemm_f32_gateup_swiglu(const GemmArgs& a, hipStream_t st);
moe_status gemm_f32_down(const GemmArgs& a, hipStream_t st);
moe_status decode_bf16(bool swiglu, const void* A, const void* B, const int32_t* off, int64_t rows, int64_t K,
                       int64_t N, int G, void* C, hipStream_t st, const int32_t* rowmap = nullptr, int kdiv = 1);

namespace {

constexpr int64_t kDecodeMaxRows = 1024;
// Decode calls with several rows per expert on average run the grouped tile
// kernel (in its 64-token shapes): from 3 rows per expert its loads of whole
// 128-byte row pieces into LDS stream the weights faster than the split-K
// MFMA form (measured on 32 experts of 2880 x 2880: gate/up at T=24, 3 rows
// per expert, 181 vs 194 us; down, in its two-stage tile of three
// workgroups per CU, 93 us at 3, 4 and 5 rows per expert against 99, 104
// and 109 us; at 2 rows the vector form's 87 us stays ahead).
constexpr int64_t kDecodeTileGateUpRows = 3;   // per expert
constexpr int64_t kDecodeTileDownRows = 3;

moe_status check_proj(const void* in, const void* w, const int32_t* offsets, int64_t rows, int64_t d, int64_t f,
                      int32_t E, moe_dtype dtype, const void* out) {
  if (rows < 0 || d <= 0 || f <= 0 || E < 1 || !valid_dtype(dtype)) return MOE_ERR_INVALID_ARG;
  if (E > kMaxE) return MOE_ERR_UNSUPPORTED;
  if (rows >= (int64_t(1) << 31)) return MOE_ERR_UNSUPPORTED;
  if (d % 64 != 0 || f % 64 != 0) return MOE_ERR_ALIGNMENT;
  if (rows == 0) return MOE_OK;
  if (!in || !w || !offsets || !out) return MOE_ERR_INVALID_ARG;
  if (!aligned16(in) || !aligned16(w) || !aligned16(out)) return MOE_ERR_ALIGNMENT;
  return MOE_OK;
}

GemmArgs proj_args(const void* in, const void* w, const int32_t* offsets, int64_t rows, int64_t K, int64_t N,
                   int32_t E, void* out) {
  GemmArgs a{};
  a.A = in;
  a.B = w;
  a.off = offsets;
  a.bias = nullptr;
  a.C = out;
  a.rows = rows;
  a.K = K;
  a.N = N;
  a.G = E;
  return a;
}

}  // namespace
}  // namespace moe

using namespace moe;

extern "C" int moe_abi_version(void) { return MOE_ABI_VERSION; }

extern "C" const char* moe_status_string(moe_status s) {
  switch (s) {
    case MOE_OK: return "ok";
    case MOE_ERR_INVALID_ARG: return "invalid argument";
    case MOE_ERR_UNSUPPORTED: return "unsupported size or option";
    case MOE_ERR_ALIGNMENT: return "misaligned pointer or size not a multiple of 64";
    case MOE_ERR_WORKSPACE: return "workspace missing or too small";
    case MOE_ERR_HIP: return "HIP launch error";
  }
  return "unknown status";
}

extern "C" moe_status moe_grouped_gemm_gateup_swiglu(const void* x_perm, const void* w_gate_up, const int32_t* offsets,
                                                     int64_t rows, int64_t d, int64_t f, int32_t E, moe_dtype dtype,
                                                     void* h, void* stream) {
  moe_status s = check_proj(x_perm, w_gate_up, offsets, rows, d, f, E, dtype, h);
  if (s != MOE_OK || rows == 0) return s;
  const GemmArgs a = proj_args(x_perm, w_gate_up, offsets, rows, d, f, E, h);
  return dtype == MOE_BF16 ? gemm_bf16_gateup_swiglu(a, as_stream(stream)) : gemm_f32_gateup_swiglu(a, as_stream(stream));
}

extern "C" moe_status moe_grouped_gemm_gateup_swiglu_gather(const void* x, const int32_t* perm, int32_t k,
                                                            const void* w_gate_up, const int32_t* offsets,
                                                            int64_t rows, int64_t d, int64_t f, int32_t E,
                                                            moe_dtype dtype, void* h, void* stream) {
  moe_status s = check_proj(x, w_gate_up, offsets, rows, d, f, E, dtype, h);
  if (s != MOE_OK) return s;
  if (k < 1 || k > kMaxK || rows % k != 0) return MOE_ERR_INVALID_ARG;
  if (rows == 0) return MOE_OK;
  if (!perm) return MOE_ERR_INVALID_ARG;
  if (dtype != MOE_BF16) return MOE_ERR_UNSUPPORTED;
  GemmArgs a = proj_args(x, w_gate_up, offsets, rows, d, f, E, h);
  a.rowmap = perm;
  a.kdiv = k;
  a.a_rows = rows / k;
  return gemm_bf16_gateup_swiglu(a, as_stream(stream));
}

extern "C" moe_status moe_grouped_gemm_down(const void* h, const void* w_down, const int32_t* offsets, int64_t rows,
                                            int64_t d, int64_t f, int32_t E, moe_dtype dtype, void* y_perm,
                                            void* stream) {
  moe_status s = check_proj(h, w_down, offsets, rows, d, f, E, dtype, y_perm);
  if (s != MOE_OK || rows == 0) return s;
  const GemmArgs a = proj_args(h, w_down, offsets, rows, f, d, E, y_perm);
  return dtype == MOE_BF16 ? gemm_bf16_down(a, as_stream(stream)) : gemm_f32_down(a, as_stream(stream));
}

extern "C" moe_status moe_decode_gateup_swiglu(const void* x_perm, const void* w_gate_up, const int32_t* offsets,
                                               int64_t rows, int64_t d, int64_t f, int32_t E, moe_dtype dtype,
                                               void* h, void* stream) {
  moe_status s = check_proj(x_perm, w_gate_up, offsets, rows, d, f, E, dtype, h);
  if (s != MOE_OK || rows == 0) return s;
  if (rows > kDecodeMaxRows) return MOE_ERR_UNSUPPORTED;
  if (dtype == MOE_F32)
    return gemm_f32_gateup_swiglu(proj_args(x_perm, w_gate_up, offsets, rows, d, f, E, h), as_stream(stream));
  if (rows >= kDecodeTileGateUpRows * E)
    return gemm_bf16_gateup_swiglu_few(proj_args(x_perm, w_gate_up, offsets, rows, d, f, E, h), as_stream(stream));
  return decode_bf16(true, x_perm, w_gate_up, offsets, rows, d, f, E, h, as_stream(stream));
}

extern "C" moe_status moe_decode_gateup_swiglu_gather(const void* x, const int32_t* perm, int32_t k,
                                                      const void* w_gate_up, const int32_t* offsets, int64_t rows,
                                                      int64_t d, int64_t f, int32_t E, moe_dtype dtype, void* h,
                                                      void* stream) {
  moe_status s = check_proj(x, w_gate_up, offsets, rows, d, f, E, dtype, h);
  if (s != MOE_OK) return s;
  if (k < 1 || k > kMaxK || rows % k != 0) return MOE_ERR_INVALID_ARG;
  if (rows == 0) return MOE_OK;
  if (!perm) return MOE_ERR_INVALID_ARG;
  if (rows > kDecodeMaxRows || dtype != MOE_BF16) return MOE_ERR_UNSUPPORTED;
  if (rows >= kDecodeTileGateUpRows * E) {
    GemmArgs a = proj_args(x, w_gate_up, offsets, rows, d, f, E, h);
    a.rowmap = perm;
    a.kdiv = k;
    a.a_rows = rows / k;
    return gemm_bf16_gateup_swiglu_few(a, as_stream(stream));
  }
  return decode_bf16(true, x, w_gate_up, offsets, rows, d, f, E, h, as_stream(stream), perm, k);
}

extern "C" moe_status moe_decode_down(const void* h, const void* w_down, const int32_t* offsets, int64_t rows,
                                      int64_t d, int64_t f, int32_t E, moe_dtype dtype, void* y_perm, void* stream) {
  moe_status s = check_proj(h, w_down, offsets, rows, d, f, E, dtype, y_perm);
  if (s != MOE_OK || rows == 0) return s;
  if (rows > kDecodeMaxRows) return MOE_ERR_UNSUPPORTED;
  if (dtype == MOE_F32)
    return gemm_f32_down(proj_args(h, w_down, offsets, rows, f, d, E, y_perm), as_stream(stream));
  if (rows >= kDecodeTileDownRows * E)
    return gemm_bf16_down_few(proj_args(h, w_down, offsets, rows, f, d, E, y_perm), as_stream(stream));
  return decode_bf16(false, h, w_down, offsets, rows, f, d, E, y_perm, as_stream(stream));
}
