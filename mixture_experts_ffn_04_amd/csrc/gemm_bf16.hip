// bf16 grouped GEMM on the gfx950 matrix cores (v_mfma_f32_32x32x16_bf16).
//
// Workgroup: 256 threads = 4 waves arranged WM x WN.  Tile: BM token rows x
// BN weight rows x 64 K.  The MFMA runs the transposed product -- weight rows
// are its 32-row operand, token rows its 32-column operand -- so each lane
// ends up with 4 consecutive output columns of one token row and writes them
// as one 8-byte (bf16) or 16-byte (fp32) store.
//
// Data movement per K step (64 elements = 128 bytes per row):
//   global -> registers: every thread loads 16-byte chunks, 8 threads per
//   row, so one instruction moves 32 full rows (coalesced 128-byte runs);
//   registers -> LDS: chunk c of row r lands at chunk position c ^ (r & 7),
//   an XOR swizzle that keeps both the row-wise stores and the MFMA
//   fragment reads (one 16-byte chunk from each of 32 consecutive rows)
//   free of bank conflicts;
//   LDS -> registers: one ds_read_b128 per 32x16 fragment.
// Two LDS buffers: the loads of step k+1 are in flight while the MFMAs of
// step k run, with one barrier per step.
#include "grouped_gemm.h"

namespace moe {

namespace {

typedef __attribute__((address_space(1))) const u32x4 gu4;   // 16 bytes in global memory

constexpr int kBK = 64;          // K per LDS stage
constexpr int kChunks = kBK / 8; // 16-byte chunks per row per stage

template <int BM, int BN, int WM, int WN, int EPI, int SN>
__global__ __launch_bounds__(256) void gemm_bf16_kernel(GemmArgs a) {
  constexpr int NT = 256;
  static_assert(WM * WN == 4, "4 waves");
  constexpr int TM = BM / WM;             // token rows per wave
  constexpr int TN = BN / WN;             // weight rows per wave
  constexpr int FM = TM / 32;             // 32-row fragments per wave (tokens)
  constexpr int FN = TN / 32;             // 32-row fragments per wave (weights)
  static_assert(FM >= 1 && FN >= 1 && TM % 32 == 0 && TN % 32 == 0, "fragment shape");
  static_assert(EPI != EPI_SWIGLU || FN % 2 == 0, "SwiGLU pairs gate and up fragments");
  constexpr int BNO = (EPI == EPI_SWIGLU) ? BN / 2 : BN;   // output columns per tile
  constexpr int ROWS_PER_LD = NT / kChunks;                // 32 rows per load instruction
  constexpr int LD_B = BN / ROWS_PER_LD;                   // weight-tile loads per thread
  constexpr int LD_A = BM / ROWS_PER_LD;                   // token-tile loads per thread
  constexpr int STAGE = (BN + BM) * kChunks;               // uint4 per LDS stage

  __shared__ u32x4 lds[2 * STAGE];

  TileLoc tl;
  if (!locate_tile<NT, BM, BNO, SN>(a, tl)) return;

  const int t = threadIdx.x;
  const int lane = t & 63;
  const int wave = t >> 6;
  const int wm = wave % WM;
  const int wn = wave / WM;
  const int64_t K = a.K;
  const int64_t N = a.N;

  // ---- global load descriptors.  Rows past the group end (tokens) or past
  // N (weights) read a valid row instead: they only feed output rows /
  // columns that the epilogue masks, so no zero-fill select is needed.
  const int ck = t & (kChunks - 1);     // chunk within the row
  const int rr = t / kChunks;           // row within a 32-row slab
  const uint16_t* Ab = static_cast<const uint16_t*>(a.A);
  const uint16_t* Bb = static_cast<const uint16_t*>(a.B) +
      static_cast<int64_t>(tl.g) * ((EPI == EPI_SWIGLU) ? 2 * N : N) * K;

  const gu4* bsrc[LD_B];
#pragma unroll
  for (int i = 0; i < LD_B; ++i) {
    const int r = i * ROWS_PER_LD + rr;          // weight-tile row
    int64_t src;
    if (EPI == EPI_SWIGLU) {
      const int half = r / (BN / 2);
      const int64_t n = tl.n0 + (r - half * (BN / 2));
      src = half * N + (n < N ? n : 0);
    } else {
      const int64_t n = tl.n0 + r;
      src = n < N ? n : 0;
    }
    bsrc[i] = (const gu4*)(Bb + src * K + ck * 8);
  }
  const gu4* asrc[LD_A];
#pragma unroll
  for (int i = 0; i < LD_A; ++i) {
    const int64_t row = static_cast<int64_t>(tl.row0) + i * ROWS_PER_LD + rr;
    asrc[i] = (const gu4*)(Ab + (row < tl.row_end ? row : tl.row0) * K + ck * 8);
  }

  u32x4 rb[LD_B], ra[LD_A];

  // k0 in elements; one K step is kBK / 8 uint4 per row
#define MOE_GLOAD(kt_)                                                                  \
  do {                                                                                  \
    const int64_t o_ = static_cast<int64_t>(kt_) * (kBK / 8);                           \
    _Pragma("unroll") for (int i = 0; i < LD_B; ++i) rb[i] = bsrc[i][o_];               \
    _Pragma("unroll") for (int i = 0; i < LD_A; ++i) ra[i] = asrc[i][o_];               \
  } while (0)
#define MOE_LSTORE(buf)                                                                 \
  do {                                                                                  \
    u32x4* s_ = lds + (buf) * STAGE;                                                    \
    _Pragma("unroll") for (int i = 0; i < LD_B; ++i) {                                  \
      const int r_ = i * ROWS_PER_LD + rr;                                              \
      s_[r_ * kChunks + (ck ^ (r_ & 7))] = rb[i];                                       \
    }                                                                                   \
    _Pragma("unroll") for (int i = 0; i < LD_A; ++i) {                                  \
      const int r_ = BN + i * ROWS_PER_LD + rr;                                         \
      s_[r_ * kChunks + (ck ^ (r_ & 7))] = ra[i];                                       \
    }                                                                                   \
  } while (0)

  // ---- fragment rows in the LDS tile
  int wrow[FN];
#pragma unroll
  for (int fn = 0; fn < FN; ++fn) {
    if (EPI == EPI_SWIGLU) {
      const int hf = fn / (FN / 2);
      wrow[fn] = hf * (BN / 2) + wn * (TN / 2) + (fn - hf * (FN / 2)) * 32;
    } else {
      wrow[fn] = wn * TN + fn * 32;
    }
  }
  const int l32 = lane & 31;
  const int khalf = lane >> 5;

  f32x16 acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j) acc[i][j] = f32x16{};

#define MOE_COMPUTE(buf)                                                                \
  do {                                                                                  \
    const u32x4* s_ = lds + (buf) * STAGE;                                              \
    _Pragma("unroll") for (int ks = 0; ks < kBK / 16; ++ks) {                           \
      const int c_ = ks * 2 + khalf;                                                    \
      bf16x8 wf[FN], tf[FM];                                                            \
      _Pragma("unroll") for (int fn = 0; fn < FN; ++fn) {                               \
        const int r_ = wrow[fn] + l32;                                                  \
        wf[fn] = __builtin_bit_cast(bf16x8, s_[r_ * kChunks + (c_ ^ (r_ & 7))]);        \
      }                                                                                 \
      _Pragma("unroll") for (int fm = 0; fm < FM; ++fm) {                               \
        const int r_ = BN + wm * TM + fm * 32 + l32;                                    \
        tf[fm] = __builtin_bit_cast(bf16x8, s_[r_ * kChunks + (c_ ^ (r_ & 7))]);        \
      }                                                                                 \
      _Pragma("unroll") for (int fm = 0; fm < FM; ++fm)                                 \
        _Pragma("unroll") for (int fn = 0; fn < FN; ++fn)                               \
          acc[fm][fn] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(wf[fn], tf[fm], acc[fm][fn], 0, 0, 0); \
    }                                                                                   \
  } while (0)

  const int nk = static_cast<int>(K / kBK);
  MOE_GLOAD(0);
  MOE_LSTORE(0);
  __syncthreads();
  for (int kt = 0; kt + 1 < nk; ++kt) {
    MOE_GLOAD(kt + 1);          // in flight during the MFMAs below
    __builtin_amdgcn_sched_barrier(0);   // keep the loads issued ahead of the MFMAs
    MOE_COMPUTE(kt & 1);
    MOE_LSTORE((kt + 1) & 1);
    __syncthreads();
  }
  MOE_COMPUTE((nk - 1) & 1);

#undef MOE_COMPUTE
#undef MOE_GLOAD
#undef MOE_LSTORE

  // ---- epilogue: lane holds output columns 8q + 4*khalf + {0..3} of token row l32
#pragma unroll
  for (int fm = 0; fm < FM; ++fm) {
    const int64_t row = static_cast<int64_t>(tl.row0) + wm * TM + fm * 32 + l32;
    if (row >= tl.row_end) continue;
    if (EPI == EPI_SWIGLU) {
      uint16_t* C = static_cast<uint16_t*>(a.C) + row * N;
#pragma unroll
      for (int fg = 0; fg < FN / 2; ++fg) {
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int64_t n = tl.n0 + wn * (TN / 2) + fg * 32 + q * 8 + khalf * 4;
          if (n >= N) continue;
          const f32x16& g = acc[fm][fg];
          const f32x16& u = acc[fm][fg + FN / 2];
          uint2 o;
          o.x = pack_bf16x2(silu(g[4 * q + 0]) * u[4 * q + 0], silu(g[4 * q + 1]) * u[4 * q + 1]);
          o.y = pack_bf16x2(silu(g[4 * q + 2]) * u[4 * q + 2], silu(g[4 * q + 3]) * u[4 * q + 3]);
          *reinterpret_cast<uint2*>(C + n) = o;
        }
      }
    } else if (EPI == EPI_STORE) {
      uint16_t* C = static_cast<uint16_t*>(a.C) + row * N;
#pragma unroll
      for (int fn = 0; fn < FN; ++fn) {
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int64_t n = tl.n0 + wn * TN + fn * 32 + q * 8 + khalf * 4;
          if (n >= N) continue;
          const f32x16& c = acc[fm][fn];
          uint2 o;
          o.x = pack_bf16x2(c[4 * q + 0], c[4 * q + 1]);
          o.y = pack_bf16x2(c[4 * q + 2], c[4 * q + 3]);
          *reinterpret_cast<uint2*>(C + n) = o;
        }
      }
    } else {  // EPI_F32B
      float* C = static_cast<float*>(a.C) + row * N;
#pragma unroll
      for (int fn = 0; fn < FN; ++fn) {
#pragma unroll
        for (int q = 0; q < 4; ++q) {
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int64_t n = tl.n0 + wn * TN + fn * 32 + q * 8 + khalf * 4 + e;
            if (n < N) C[n] = acc[fm][fn][4 * q + e] + (a.bias ? a.bias[n] : 0.0f);
          }
        }
      }
    }
  }
}

template <int BM, int BN, int WM, int WN, int EPI, int SN>
moe_status launch(const GemmArgs& a, hipStream_t st) {
  constexpr int BNO = (EPI == EPI_SWIGLU) ? BN / 2 : BN;
  const int64_t grid = grouped_tile_bound(a.rows, a.G, BM, a.N, BNO);
  if (grid <= 0) return MOE_OK;
  if (grid > 0x7fffffff) return MOE_ERR_UNSUPPORTED;
  hipLaunchKernelGGL((gemm_bf16_kernel<BM, BN, WM, WN, EPI, SN>), dim3(static_cast<unsigned>(grid)),
                     dim3(256), 0, st, a);
  return launch_status();
}

}  // namespace

// Entry points used by the C ABI (argument checks are done by the caller).
moe_status gemm_bf16_gateup_swiglu(const GemmArgs& a, hipStream_t st) {
  return launch<128, 256, 2, 2, EPI_SWIGLU, 8>(a, st);
}

moe_status gemm_bf16_down(const GemmArgs& a, hipStream_t st) {
  return launch<128, 256, 2, 2, EPI_STORE, 8>(a, st);
}

moe_status gemm_bf16_logits(const GemmArgs& a, hipStream_t st) {
  if (a.N <= 64) return launch<128, 64, 4, 1, EPI_F32B, 1>(a, st);
  return launch<128, 256, 2, 2, EPI_F32B, 1>(a, st);
}

}  // namespace moe
