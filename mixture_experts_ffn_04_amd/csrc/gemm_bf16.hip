// bf16 grouped GEMMs on the gfx950 matrix cores (v_mfma_f32_32x32x16_bf16):
// the expert projections, and the router logits for many experts and tokens.
//
// gemm_bf16_dtl_kernel runs the transposed product -- weight rows are the
// MFMA's 32-row operand, token rows its 32-column operand -- so each lane
// ends up with 4 consecutive output columns of one token row and writes
// them as one 8-byte (bf16) or four 4-byte (fp32) stores.  Both operands
// are K-contiguous rows, so a fragment (32 rows x 16 K) is one ds_read_b128
// per lane.  Buffer loads go straight into LDS (no register staging); three
// weight stages and two token stages of 64 K-elements, so weight loads run
// two stages and token loads one stage ahead of the MFMAs (tiles of more
// than 256 token rows, which absorb an expert's small remainder, keep two
// stages of each).
//
// LDS layout: tile row r holds the 64 elements of one weight or token row
// as 8 16-byte chunks; chunk c is stored at position c ^ swz(r).  gfx950
// serves a ds_read_b128 16 lanes (256 bytes, all 64 banks) per cycle; a
// fragment read takes one chunk from each of 32 consecutive rows, and swz
// spreads every group of 16 such rows over all 64 banks (and keeps the
// row-wise writes conflict free).
#include "grouped_gemm.h"

namespace moe {

namespace {

typedef __attribute__((address_space(1))) const u32x4 gu4;   // 16 bytes in global memory
typedef __attribute__((address_space(3))) void lds_void;

// raw buffer descriptor word 3 for gfx9-family untyped 32-bit accesses
constexpr int kBufFlags = 0x00020000;

// 128-byte tile rows (CH = 8 chunks): rows r and r+1 sit in different
// 128-byte bank halves, and the 8 same-parity rows among 16 need 8 distinct
// positions.
template <int CH>
__host__ __device__ __forceinline__ int swz(int r) {
  static_assert(CH == 8, "128-byte tile rows");
  return (r & 7) ^ ((r >> 3) & 1);
}

// Scheduling groups (sched_group_barrier masks): each K slice's MFMAs are
// interleaved one-to-one with the LDS reads of the next slice, so LDS
// latency hides under MFMA execution.
#define MOE_SG(mask, n) __builtin_amdgcn_sched_group_barrier(mask, n, 0)
#define MOE_SG_MFMA 0x008
#define MOE_SG_DSR 0x100

// One LDS stage of KS 16-wide K slices: the NR fragment reads of the first
// slice, then per slice its NM MFMAs paired with the reads of the next
// slice.
template <int NR, int NM, int KS>
__device__ __forceinline__ void sched_stage() {
  constexpr int P = NR < NM ? NR : NM;
  MOE_SG(MOE_SG_DSR, NR);
#pragma unroll
  for (int ks = 0; ks + 1 < KS; ++ks) {
#pragma unroll
    for (int i = 0; i < P; ++i) {
      MOE_SG(MOE_SG_MFMA, 1);
      MOE_SG(MOE_SG_DSR, 1);
    }
    if (NM > P) MOE_SG(MOE_SG_MFMA, NM - P);
    if (NR > P) MOE_SG(MOE_SG_DSR, NR - P);
  }
  MOE_SG(MOE_SG_MFMA, NM);
}

// The NF_ x FN MFMAs of one K slice on fragments wf_ (weights) and tf_
// (tokens).
#define MOE_MFMAS(wf_, tf_, NF_)                                                        \
  do {                                                                                  \
    _Pragma("unroll") for (int fm = 0; fm < (NF_); ++fm)                                \
      _Pragma("unroll") for (int fn = 0; fn < FN; ++fn)                                 \
        acc[fm][fn] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(wf_[fn], tf_[fm], acc[fm][fn], 0, 0, 0); \
  } while (0)

// Fragment row of each of the FN weight fragments of wave column wn.  With
// SwiGLU the tile holds BN/2 gate rows then the matching BN/2 up rows, and a
// wave takes the same columns from both halves.
template <int EPI, int BN, int TN, int FN>
__device__ __forceinline__ void weight_frag_rows(int wn, int* wrow) {
#pragma unroll
  for (int fn = 0; fn < FN; ++fn) {
    if (EPI == EPI_SWIGLU) {
      const int hf = fn / (FN / 2);
      wrow[fn] = hf * (BN / 2) + wn * (TN / 2) + (fn - hf * (FN / 2)) * 32;
    } else {
      wrow[fn] = wn * TN + fn * 32;
    }
  }
}

// Epilogue: lane holds output columns 8q + 4*khalf + {0..3} of token row l32
// in each 32x32 accumulator block.
template <int EPI, int FM, int FN, int TM, int TN>
__device__ __forceinline__ void store_tile(const GemmArgs& a, const TileLoc& tl, const f32x16 (&acc)[FM][FN],
                                           int wm, int wn, int l32, int khalf) {
  const int64_t N = a.N;
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

// ---------------------------------------------------------------------------
// Direct-to-LDS kernel (expert projections).
//
// Synchronisation per stage: s_waitcnt vmcnt(n) (this wave's loads of the
// stage about to be consumed have landed; only the n youngest loads may
// still be in flight) and lgkmcnt(0) (this wave's LDS reads of the buffers
// about to be refilled are complete), then s_barrier.  This is not the
// __syncthreads() fence, which would wait for every outstanding LDS DMA.
// After the loop all DMA is drained before the epilogue, so nothing lands
// in LDS after the workgroup ends.

template <int VM>
__device__ __forceinline__ void wait_stage_barrier() {
  static_assert(VM < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((VM & 15) | (7 << 4) | (0 << 8) | ((VM >> 4) << 14));
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

__device__ __forceinline__ void drain_vm() {
  __builtin_amdgcn_s_waitcnt(0 | (7 << 4) | (15 << 8) | (0 << 14));   // vmcnt(0)
  asm volatile("" ::: "memory");
}

// One LDS DMA: 64 lanes x 16 bytes from buffer rs at per-lane byte offset
// voff (+ soff) into LDS [lds_addr, lds_addr + 1024).  Written as asm so the
// compiler does not add its own conservative "all LDS DMA done" wait before
// later LDS reads of another stage; the kernel waits explicitly (vmcnt)
// before the barrier that publishes a stage.  The instruction has no
// register outputs.  Nothing else in these kernels uses m0.
__device__ __forceinline__ void lds_dma16(__amdgpu_buffer_rsrc_t rs, int voff, int soff, unsigned lds_addr) {
  asm volatile("s_mov_b32 m0, %3\n\ts_nop 0\n\tbuffer_load_dwordx4 %0, %1, %2 offen lds"
               :: "v"(voff), "s"(rs), "s"(soff), "s"(lds_addr) : "memory", "m0");
}

__device__ __forceinline__ unsigned lds_addr_of(const void* p) {
  return static_cast<unsigned>(reinterpret_cast<uintptr_t>((const lds_void*)p));
}

// SP: the DMA instructions of a stage are spread over the fragment reads of
// its first SP K slices rather than issued in one burst.
// Epilogue through LDS (bf16 outputs): every lane writes its 4-column
// pieces into a row-major copy of the output tile in LDS (chunk c of row r
// at c ^ (r % NCH), which spreads a fragment's 32 rows over the banks),
// then every thread stores whole 16-byte chunks of whole rows, so each
// store instruction covers full rows of C instead of 16-byte pieces of 32
// rows.  smem holds BM * BNO * 2 bytes; the caller has made sure no wave
// still reads or loads into it.
template <int EPI, int FM, int FN, int TM, int TN, int BM, int BNO, int NT>
__device__ __forceinline__ void store_tile_lds(const GemmArgs& a, const TileLoc& tl, const f32x16 (&acc)[FM][FN],
                                               int wm, int wn, int l32, int khalf, char* smem) {
  constexpr int RB = BNO * 2;          // bytes per tile row
  constexpr int NCH = RB / 16;         // 16-byte chunks per tile row
#pragma unroll
  for (int fm = 0; fm < FM; ++fm) {
    const int r = wm * TM + fm * 32 + l32;
    char* row = smem + r * RB;
    const int sz = r % NCH;
    if (EPI == EPI_SWIGLU) {
#pragma unroll
      for (int fg = 0; fg < FN / 2; ++fg) {
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int ch = (wn * (TN / 2) + fg * 32 + q * 8) / 8;
          const f32x16& g = acc[fm][fg];
          const f32x16& u = acc[fm][fg + FN / 2];
          uint2 o;
          o.x = pack_bf16x2(silu(g[4 * q + 0]) * u[4 * q + 0], silu(g[4 * q + 1]) * u[4 * q + 1]);
          o.y = pack_bf16x2(silu(g[4 * q + 2]) * u[4 * q + 2], silu(g[4 * q + 3]) * u[4 * q + 3]);
          *reinterpret_cast<uint2*>(row + ((ch ^ sz) * 16) + khalf * 8) = o;
        }
      }
    } else {
#pragma unroll
      for (int fn = 0; fn < FN; ++fn) {
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int ch = (wn * TN + fn * 32 + q * 8) / 8;
          const f32x16& c = acc[fm][fn];
          uint2 o;
          o.x = pack_bf16x2(c[4 * q + 0], c[4 * q + 1]);
          o.y = pack_bf16x2(c[4 * q + 2], c[4 * q + 3]);
          *reinterpret_cast<uint2*>(row + ((ch ^ sz) * 16) + khalf * 8) = o;
        }
      }
    }
  }
  __syncthreads();
  const int nrows = min(tl.row_end - tl.row0, BM);
  const int64_t N = a.N;
  uint16_t* C = static_cast<uint16_t*>(a.C) + static_cast<int64_t>(tl.row0) * N + tl.n0;
#pragma unroll 4
  for (int c = threadIdx.x; c < BM * NCH; c += NT) {
    const int r = c / NCH;
    const int ch = c - r * NCH;
    if (r >= nrows) break;                     // rows past the tile's rows: never stored (c only grows)
    if (tl.n0 + ch * 8 >= N) continue;          // columns past N (N is a multiple of 64)
    const u32x4 v = *reinterpret_cast<const u32x4*>(smem + r * RB + ((ch ^ (r % NCH)) * 16));
    *reinterpret_cast<u32x4*>(C + static_cast<int64_t>(r) * N + ch * 8) = v;
  }
}

// Per-lane byte offsets (from the tile's buffer descriptors) and LDS byte
// offsets inside a stage of a wave's NL load instructions.  The first NX
// fill token rows of the wave's own row block, instruction i its token
// fragment i (rows tm * wm + RPI (wn + WN i) ...), so the waves that read a
// fragment are the ones that load it; the rest fill RPI weight rows each.
// Lane t covers row +t/CH, LDS slot t%CH and global chunk (t%CH) ^ swz(row).
// With a row map, token rows past the tile's last row read row 0 (their
// results are never stored).
template <int EPI, int BN, int CH, int RPI, int NW, int WN, int NX, int NL>
__host__ __device__ __forceinline__ void dma_offsets(const GemmArgs& a, const TileLoc& tl, int64_t rowb, bool gather, int wave,
                                            int wm, int wn, int lane, int tm, int (&voff)[NL], int (&dst)[NL]) {
  const int64_t N = a.N;
#pragma unroll
  for (int i = 0; i < NL; ++i) {
    const bool tok = i < NX;
    const int row0 = tok ? wm * tm + RPI * (wn + WN * i) : RPI * (wave + NW * (i - NX));
    const int r = row0 + lane / CH;
    const int c = (lane % CH) ^ swz<CH>(r);
    int64_t off;
    if (!tok) {
      if (EPI == EPI_SWIGLU) {
        const int half = r / (BN / 2);
        off = (half * N + tl.n0 + (r - half * (BN / 2))) * rowb;
      } else {
        off = static_cast<int64_t>(r) * rowb;
      }
    } else if (gather) {
      const int grow = tl.row0 + r;
      const int src = grow < tl.row_end ? clamp_off(a.rowmap[grow], static_cast<int>(a.rows) - 1) / a.kdiv : 0;
      off = static_cast<int64_t>(src) * rowb;
    } else {
      off = static_cast<int64_t>(r) * rowb;
    }
    voff[i] = static_cast<int>(off) + c * 16;
    dst[i] = row0 * CH * 16;
  }
}

// The tile kernel's shape constants: wave layout, fragments, load
// instructions per wave and stage, and LDS stage sizes (16-byte units).
template <int BM, int BN, int WM, int WN, int EPI, int BK, int WS = 3>
struct DtlShape {
  static constexpr int NW = WM * WN;
  static constexpr int NT = 64 * NW;
  static constexpr int TM = BM / WM, TN = BN / WN;
  static constexpr int FM = TM / 32, FN = TN / 32;
  static constexpr int CH = BK / 8;                   // 16-byte chunks per tile row
  static constexpr int KS = BK / 16;                  // 16-wide K slices per stage
  static constexpr int RPI = 64 / CH;                 // tile rows per 1 KB load instruction
  static constexpr int BNO = (EPI == EPI_SWIGLU) ? BN / 2 : BN;
  static constexpr int LB = BN / (RPI * NW);          // weight load instructions per wave per stage
  static constexpr int LX = BM / (RPI * NW);          // token load instructions
  static constexpr int LPS = LB + LX;
  static constexpr int WSTG = BN * CH, XSTG = BM * CH;   // units per weight / token stage
  static constexpr int LDS_UNITS = WS * WSTG + 2 * XSTG;   // WS weight stages, 2 token stages
  // Fat tiles: an expert's last remainder of up to kFatExtraRows rows shared
  // out over its other row tiles, BMF = BM + kFatExtraRows rows at most,
  // with two stages of both operands (three weight stages no longer fit).
  static constexpr bool FAT_OK = BM == 256 && WM == 2 && EPI != EPI_F32B;
  static constexpr int BMF = BM + kFatExtraRows, TMF = BMF / WM, FMF = TMF / 32;
  static constexpr int LXF = BMF / (RPI * NW), LPF = LB + LXF;
  static constexpr int XSTGF = BMF * CH;
};

// Byte offsets from a.B and a.A of the tile's two buffer descriptors, their
// extents (num_records), and the tile's valid token rows.  Weights: expert
// g's rows (gate/up: all 2N rows; down: from the tile's first output
// column on).  Tokens: the tile's own rows of A, or with a row map all of A.
// num_records is the valid extent, so rows past N or past the tile's last
// token row read as zero (hardware bounds check).
struct TileBuffers {
  int64_t wbase;
  int wrecords;
  int64_t abase;
  int arecords;
  int vrows;
};

template <int EPI, int BM, bool FAT_OK, int BMF>
__host__ __device__ __forceinline__ TileBuffers tile_buffers(const GemmArgs& a, const TileLoc& tl) {
  const int64_t N = a.N;
  const int64_t rowb = a.K * 2;                       // bytes per row
  TileBuffers b;
  b.wbase = static_cast<int64_t>(tl.g) * ((EPI == EPI_SWIGLU) ? 2 * N : N) * rowb;
  if (EPI == EPI_SWIGLU) {
    b.wrecords = static_cast<int>(2 * N * rowb);      // gate rows [0, N), up rows [N, 2N)
  } else {
    b.wbase += tl.n0 * rowb;
    b.wrecords = static_cast<int>((N - tl.n0) * rowb);
  }
  const bool gather = a.rowmap != nullptr;
  b.abase = gather ? 0 : static_cast<int64_t>(tl.row0) * rowb;
  b.vrows = tl.row_end - tl.row0;                     // at most BM, or BMF for a fat tile
  const int cap = FAT_OK ? BMF : BM;
  b.arecords = gather ? static_cast<int>(a.a_rows * rowb) : static_cast<int>((b.vrows < cap ? b.vrows : cap) * rowb);
  return b;
}

// Fragment reads of K slice ks (16 wide) -- the FN weight fragments from
// weight stage sw_ and the first NF_ token fragments from token stage sx_
// (their MFMAs are MOE_MFMAS).
#define MOE_DTL_FRAGS(wf_, tf_, sw_, sx_, ks_, NF_)                                     \
  do {                                                                                  \
    const int c_ = ((ks_) * 2 + khalf) ^ sw;                                            \
    _Pragma("unroll") for (int fn = 0; fn < FN; ++fn)                                   \
      wf_[fn] = __builtin_bit_cast(bf16x8, (sw_)[(wrow[fn] + l32) * CH + c_]);          \
    _Pragma("unroll") for (int fm = 0; fm < (NF_); ++fm)                                \
      tf_[fm] = __builtin_bit_cast(bf16x8, (sx_)[(wm * TM + fm * 32 + l32) * CH + c_]); \
  } while (0)

// One tile per workgroup, in the order of locate_tile.
//
// Stages: weight rows come from the Infinity Cache or HBM (each weight tile
// is shared by only the few row tiles of its expert), token rows mostly
// from L2 (shared by every column tile of the expert).  So the 160 KB of
// LDS hold three weight stages and two token stages of BK = 64: the loads
// of stage k+2's weights and stage k+1's tokens are issued during stage k.
// Per stage each wave issues its token loads before its weight loads, so
// s_waitcnt vmcnt(LB) at the top of stage k (only stage k+1's weights may
// still be in flight) means stage k's tokens and weights have landed; the
// s_barrier after it publishes them and also tells every wave that the
// buffers of stage k-1, refilled during stage k, are no longer read.
// WS = 2 (two stages of both operands, a smaller LDS footprint so that
// more workgroups share a CU): each stage's loads are issued right after
// the barrier of the stage before, which waits for all of the wave's loads.
// The waves-per-EU bound asks for three such workgroups per CU.
template <int BM, int BN, int WM, int WN, int EPI, int SN, int BK, int SP, int LDS_EPI, int WS>
__global__ __launch_bounds__(64 * WM * WN, (WS == 2 ? 3 : 1) * WM * WN / 4) void gemm_bf16_dtl_kernel(GemmArgs a) {
#if defined(__HIP_DEVICE_COMPILE__)   // the body uses device-only types; the host pass needs only the stub
  static_assert(WS == 2 || WS == 3, "weight stages");
  static_assert(WS == 3 || !(BM == 256 && WM == 2 && EPI != EPI_F32B), "fat tiles keep three weight stages");
  typedef DtlShape<BM, BN, WM, WN, EPI, BK, WS> S;
  constexpr int NW = S::NW, NT = S::NT, TM = S::TM, TN = S::TN, FM = S::FM, FN = S::FN;
  static_assert(FM >= 1 && FN >= 1 && TM % 32 == 0 && TN % 32 == 0, "fragment shape");
  static_assert(EPI != EPI_SWIGLU || FN % 2 == 0, "SwiGLU pairs gate and up fragments");
  static_assert(BK == 64, "stage width");
  static_assert(FM <= 4, "active-fragment specialisations cover up to 4 token fragments");
  constexpr int CH = S::CH, KS = S::KS, RPI = S::RPI, BNO = S::BNO;
  static_assert(BN % (RPI * NW) == 0 && BM % (RPI * NW) == 0, "rows per wave");
  constexpr int LB = S::LB, LX = S::LX, LPS = S::LPS;
  constexpr int WSTG = S::WSTG, XSTG = S::XSTG, LDS_UNITS = S::LDS_UNITS;
  static_assert(LDS_UNITS * 16 <= 160 * 1024, "LDS");
  static_assert(locate_scratch_ints(NT) * 4 <= LDS_UNITS * 16, "tile scan scratch fits the stages");
  static_assert(SP >= 1 && SP <= KS && LPS % SP == 0, "DMA spread");
  static_assert(RPI * WN == 32 && LX == FM, "token load instruction i fills token fragment i of the wave's row block");
  constexpr bool FAT_OK = S::FAT_OK;
  constexpr int BMF = S::BMF, TMF = S::TMF, FMF = S::FMF, LXF = S::LXF, LPF = S::LPF, XSTGF = S::XSTGF;

  __shared__ u32x4 lds[LDS_UNITS];

  TileLoc tl;
  if (!locate_tile<NT, BM, BNO, SN>(a, tl, reinterpret_cast<int*>(lds))) return;
  __syncthreads();                                    // the scratch is read by all before the loads overwrite it

  const int t = threadIdx.x;
  const int lane = t & 63;
  const int wave = __builtin_amdgcn_readfirstlane(t >> 6);
  // Waves w and w+4 share a SIMD.  Row block wm = wave / WN puts waves of
  // different row blocks on each SIMD, so when the tile's last token rows
  // are missing (the ragged end of an expert's group) the MFMAs a wave skips
  // shorten its SIMD's work instead of idling it.
  const int wm = wave / WN;
  const int wn = wave % WN;
  const int64_t K = a.K;
  const int64_t N = a.N;
  // token fragments of this wave holding at least one row of the tile
  const int trows = min(tl.row_end - tl.row0, BM) - wm * TM;
  const int nfm = trows <= 0 ? 0 : min(FM, (trows + 31) / 32);

  // Buffer descriptors based at the tile's first weight row and first token
  // row (or all of A with a row map), so every per-lane offset stays a
  // small 32-bit byte offset (tile_buffers).
  const int64_t rowb = K * 2;                          // bytes per row
  const bool gather = a.rowmap != nullptr;
  const TileBuffers tb = tile_buffers<EPI, BM, FAT_OK, BMF>(a, tl);
  const int vrows = tb.vrows;
  const __amdgpu_buffer_rsrc_t wrs = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<char*>(static_cast<const char*>(a.B) + tb.wbase), 0, tb.wrecords, kBufFlags);
  const __amdgpu_buffer_rsrc_t ars = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<char*>(static_cast<const char*>(a.A) + tb.abase), 0, tb.arecords, kBufFlags);

  if constexpr (FAT_OK) {
    if (vrows > BM) {
      static_assert(2 * WSTG + 2 * XSTGF <= LDS_UNITS, "fat tile stages fit");
      static_assert(!LDS_EPI || LDS_UNITS * 16 >= BMF * BNO * 2, "fat output tile fits the stages");
      // Token instruction i of a wave fills fragment i of its 160-row block.
      int voff[LPF];
      int dst[LPF];
      dma_offsets<EPI, BN, CH, RPI, NW, WN, LXF, LPF>(a, tl, rowb, gather, wave, wm, wn, lane, TMF, voff, dst);
      const unsigned ldsw = lds_addr_of(lds);
      const unsigned ldsxf = ldsw + 2u * WSTG * 16u;
      auto stage_dma = [&](int b, int k) {
#pragma unroll
        for (int i = 0; i < LXF; ++i)
          lds_dma16(ars, voff[i], k * (BK * 2),
                    __builtin_amdgcn_readfirstlane(ldsxf + static_cast<unsigned>(b) * (XSTGF * 16) + dst[i]));
#pragma unroll
        for (int i = LXF; i < LPF; ++i)
          lds_dma16(wrs, voff[i], k * (BK * 2),
                    __builtin_amdgcn_readfirstlane(ldsw + static_cast<unsigned>(b) * (WSTG * 16) + dst[i]));
      };
      int wrow[FN];
      weight_frag_rows<EPI, BN, TN, FN>(wn, wrow);
      const int l32 = lane & 31;
      const int khalf = lane >> 5;
      const int sw = swz<CH>(l32);
      f32x16 acc[FMF][FN];
#pragma unroll
      for (int i = 0; i < FMF; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j) acc[i][j] = f32x16{};
      const int nk = static_cast<int>(K / BK);
      const int last = nk - 1;
      // half 0 is full; half 1 holds more than 96 rows, so 4 or 5 fragments
      const int nff = min(FMF, (vrows - wm * TMF + 31) / 32);
      stage_dma(0, 0);
      // Stage kt in buffers kt & 1: wait for this wave's loads of stage kt,
      // then the barrier publishes them and frees the buffers of stage kt-1
      // for stage kt+1's loads.
#define MOE_FAT_LOOP(NF_)                                                                       \
      for (int kt = 0; kt < nk; ++kt) {                                                         \
        wait_stage_barrier<0>();                                                                \
        stage_dma((kt + 1) & 1, kt + 1 < last ? kt + 1 : last);                                 \
        const u32x4* sw_ = lds + (kt & 1) * WSTG;                                               \
        const u32x4* sx_ = lds + 2 * WSTG + (kt & 1) * XSTGF;                                   \
        _Pragma("unroll") for (int ks = 0; ks < KS; ++ks) {                                     \
          const int c_ = (ks * 2 + khalf) ^ sw;                                                 \
          bf16x8 wf[FN], tf[FMF];                                                               \
          _Pragma("unroll") for (int fn = 0; fn < FN; ++fn)                                     \
            wf[fn] = __builtin_bit_cast(bf16x8, sw_[(wrow[fn] + l32) * CH + c_]);               \
          _Pragma("unroll") for (int fm = 0; fm < (NF_); ++fm)                                  \
            tf[fm] = __builtin_bit_cast(bf16x8, sx_[(wm * TMF + fm * 32 + l32) * CH + c_]);     \
          MOE_MFMAS(wf, tf, (NF_));                                                             \
        }                                                                                       \
      }
      if (nff == FMF) {
        MOE_FAT_LOOP(FMF)
      } else {
        MOE_FAT_LOOP(FMF - 1)
      }
#undef MOE_FAT_LOOP
      drain_vm();
      if (LDS_EPI) {
        __syncthreads();
        store_tile_lds<EPI, FMF, FN, TMF, TN, BMF, BNO, NT>(a, tl, acc, wm, wn, l32, khalf, reinterpret_cast<char*>(lds));
      } else {
        store_tile<EPI, FMF, FN, TMF, TN>(a, tl, acc, wm, wn, l32, khalf);
      }
      return;
    }
  }

  // Load instruction i of this wave: the first LX fill its token fragments,
  // the rest weight rows (dma_offsets).
  int voff[LPS];
  int dst[LPS];
  dma_offsets<EPI, BN, CH, RPI, NW, WN, LX, LPS>(a, tl, rowb, gather, wave, wm, wn, lane, TM, voff, dst);
  const unsigned ldsw = lds_addr_of(lds);                          // weight stages 0 .. WS-1
  const unsigned ldsx = ldsw + static_cast<unsigned>(WS) * WSTG * 16u;   // token stages 0..1

  // Load instruction i for weight stage kw_ into weight buffer wb_, or token
  // stage kx_ into token buffer xb_.
#define MOE_DTL_DMA(i_, wb_, kw_, xb_, kx_)                                                          \
  do {                                                                                              \
    if ((i_) < LX)                                                                                  \
      lds_dma16(ars, voff[i_], (kx_) * (BK * 2),                                                    \
                __builtin_amdgcn_readfirstlane(ldsx + static_cast<unsigned>(xb_) * (XSTG * 16) + dst[i_])); \
    else                                                                                            \
      lds_dma16(wrs, voff[i_], (kw_) * (BK * 2),                                                    \
                __builtin_amdgcn_readfirstlane(ldsw + static_cast<unsigned>(wb_) * (WSTG * 16) + dst[i_])); \
  } while (0)

  int wrow[FN];
  weight_frag_rows<EPI, BN, TN, FN>(wn, wrow);
  const int l32 = lane & 31;
  const int khalf = lane >> 5;
  const int sw = swz<CH>(l32);                  // every fragment starts on a multiple of 16 rows

  f32x16 acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j) acc[i][j] = f32x16{};

  const int nk = static_cast<int>(K / BK);
  const int last = nk - 1;
  if constexpr (WS == 2) {
    // Stage kt in buffers kt & 1; token fragments at or past the row
    // block's active ones are never read, so their loads are left out.
    auto stage_dma = [&](int b, int k) {
#pragma unroll
      for (int i = 0; i < LPS; ++i)
        if (i >= LX || i < nfm) MOE_DTL_DMA(i, b, k, b, k);
    };
    stage_dma(0, 0);
#define MOE_TWO_LOOP(NF_)                                                               \
    for (int kt = 0; kt < nk; ++kt) {                                                   \
      wait_stage_barrier<0>();                                                          \
      stage_dma((kt + 1) & 1, kt + 1 < last ? kt + 1 : last);                           \
      const u32x4* sw_ = lds + (kt & 1) * WSTG;                                         \
      const u32x4* sx_ = lds + 2 * WSTG + (kt & 1) * XSTG;                              \
      _Pragma("unroll") for (int ks = 0; ks < KS; ++ks) {                               \
        bf16x8 wf_t[FN], tf_t[FM];                                                      \
        MOE_DTL_FRAGS(wf_t, tf_t, sw_, sx_, ks, NF_);                                   \
        MOE_MFMAS(wf_t, tf_t, NF_);                                                     \
      }                                                                                 \
    }
    if (nfm == FM) {
      MOE_TWO_LOOP(FM)
    } else if (nfm == 0) {
      MOE_TWO_LOOP(0)
    } else if (nfm == 1) {
      MOE_TWO_LOOP(1)
    } else if (nfm == 2) {
      MOE_TWO_LOOP(FM > 2 ? 2 : FM)
    } else {
      MOE_TWO_LOOP(FM > 3 ? 3 : FM)
    }
#undef MOE_TWO_LOOP
  } else {
  // Prologue: tokens and weights of stage 0, then the weights of stage 1
  // (stages past the end are clamped: extra loads of valid memory, never
  // consumed).
#pragma unroll
  for (int i = 0; i < LPS; ++i) MOE_DTL_DMA(i, 0, 0, 0, 0);
#pragma unroll
  for (int i = LX; i < LPS; ++i) MOE_DTL_DMA(i, 1, (1 < last ? 1 : last), 0, 0);
  int cw = 0, cx = 0;                           // weight and token buffers of stage kt
  // Part p < SP of the loads of one stage (tokens first), issued after the
  // fragment reads of K slice p.  Token fragments at or past NF_ are never
  // read by the waves that load them, so their loads are left out.
#define MOE_DTL_PART(p_, NF_)                                                           \
  if ((p_) < SP) {                                                                      \
    _Pragma("unroll") for (int i = (p_) * (LPS / SP); i < ((p_) + 1) * (LPS / SP); ++i) \
      if (i >= LX || i < (NF_)) MOE_DTL_DMA(i, nbw, kw, nbx, kx);                       \
  }
  // All KS slices of one stage, the reads of slice ks+1 in flight during the
  // MFMAs of slice ks, the stage's loads spread over its first SP slices.
#define MOE_DTL_COMPUTE(NF_)                                                            \
  do {                                                                                  \
    const u32x4* sw_ = lds + cw * WSTG;                                                 \
    const u32x4* sx_ = lds + 3 * WSTG + cx * XSTG;                                      \
    bf16x8 wf0[FN], tf0[FM], wf1[FN], tf1[FM];                                          \
    MOE_DTL_FRAGS(wf0, tf0, sw_, sx_, 0, NF_);                                          \
    MOE_DTL_PART(0, NF_);                                                               \
    _Pragma("unroll") for (int ks = 0; ks < KS; ks += 2) {                              \
      MOE_DTL_FRAGS(wf1, tf1, sw_, sx_, ks + 1, NF_);                                   \
      MOE_DTL_PART(ks + 1, NF_);                                                        \
      MOE_MFMAS(wf0, tf0, NF_);                                                     \
      if (ks + 2 < KS) {                                                                \
        MOE_DTL_FRAGS(wf0, tf0, sw_, sx_, ks + 2, NF_);                                 \
        MOE_DTL_PART(ks + 2, NF_);                                                      \
      }                                                                                 \
      MOE_MFMAS(wf1, tf1, NF_);                                                     \
    }                                                                                   \
  } while (0)
  // The K loop, specialised on the number of active token fragments (every
  // wave takes part in the loads and barriers, whatever its share).  Stage
  // kt refills the buffers of stage kt-1: tokens of stage kt+1 and weights
  // of stage kt+2.
#define MOE_DTL_LOOP(NF_)                                                               \
  for (int kt = 0; kt < nk; ++kt) {                                                     \
    wait_stage_barrier<LB>();                                                           \
    const int kx = kt + 1 < last ? kt + 1 : last;                                       \
    const int kw = kt + 2 < last ? kt + 2 : last;                                       \
    const int nbx = cx ^ 1;                                                             \
    const int nbw = cw == 0 ? 2 : cw - 1;                                               \
    if ((NF_) > 0) {                                                                    \
      MOE_DTL_COMPUTE((NF_));                                                           \
      sched_stage<FN + (NF_), FN * ((NF_) > 0 ? (NF_) : 1), KS>();                \
    } else {                                                                            \
      _Pragma("unroll") for (int i = LX; i < LPS; ++i) MOE_DTL_DMA(i, nbw, kw, nbx, kx); \
    }                                                                                   \
    cw = cw == 2 ? 0 : cw + 1;                                                          \
    cx ^= 1;                                                                            \
  }
  if (nfm == FM) {
    MOE_DTL_LOOP(FM)
  } else if (nfm == 0) {
    MOE_DTL_LOOP(0)
  } else if (nfm == 1) {
    MOE_DTL_LOOP(1)
  } else if (nfm == 2) {
    MOE_DTL_LOOP(FM > 2 ? 2 : FM)
  } else {
    MOE_DTL_LOOP(FM > 3 ? 3 : FM)
  }
  }
  drain_vm();
#undef MOE_DTL_LOOP
#undef MOE_DTL_COMPUTE
#undef MOE_DTL_PART
#undef MOE_DTL_DMA

  if (LDS_EPI) {
    static_assert(!LDS_EPI || LDS_UNITS * 16 >= BM * BNO * 2, "output tile fits the stages");
    __syncthreads();                             // every wave is past its last LDS read and DMA
    store_tile_lds<EPI, FM, FN, TM, TN, BM, BNO, NT>(a, tl, acc, wm, wn, l32, khalf, reinterpret_cast<char*>(lds));
  } else {
    store_tile<EPI, FM, FN, TM, TN>(a, tl, acc, wm, wn, l32, khalf);
  }
#endif
}
#undef MOE_DTL_FRAGS

#undef MOE_MFMAS

// Fat tiles only for K >= kFatMinK.  Measured, outputs bit-identical: gate/up
// of 8 experts of ~1024 rows at K = 4096 +2.9% (1.630 -> 1.584 ms), their
// down projection at K = 14336 +2% over the best smaller row tiles, and
// gate/up of 256 Zipf-loaded experts at K = 7168 +1%; at K = 2048 (128
// Zipf-loaded experts, gate/up; 256 experts, down) flat to 4% slower, where
// a fat tile's longer critical path and its two-stage pipeline cost more
// than the remainder tile it replaces.
constexpr int64_t kFatMinK = 4096;

// Short K loops walk the tile order in four interleaved quarters.
constexpr int64_t kQuarterMaxK = 1024;

template <int BM, int BN, int WM, int WN, int EPI, int SN, int BK, int SP = 1, int LDS_EPI = 0, int WS = 3>
moe_status launch_dtl(const GemmArgs& a, hipStream_t st) {
  constexpr int BNO = (EPI == EPI_SWIGLU) ? BN / 2 : BN;
  // A launch of fewer than kAdaptRounds rounds of full tiles may pick
  // smaller row tiles on the device; its grid then covers the smallest.
  GemmArgs b = a;
  b.adapt_rows = 0;
  b.fat_rows = (BM == 256 && WM == 2 && EPI != EPI_F32B && a.K >= kFatMinK) ? 1 : 0;   // fat tiles: fewer tiles
  b.quarters = (EPI != EPI_F32B && a.K < kQuarterMaxK) ? 1 : 0;
  int64_t grid = grouped_tile_bound(a.rows, a.G, BM, a.N, BNO);
  if (EPI != EPI_F32B && BM >= 32 * kRowChoices && grid < int64_t(kAdaptRounds) * kComputeUnits) {
    b.adapt_rows = 1;
    grid = grouped_tile_bound(a.rows, a.G, BM - 32 * (kRowChoices - 1), a.N, BNO);
  }
  if (grid <= 0) return MOE_OK;
  if (grid > 0x7fffffff) return MOE_ERR_UNSUPPORTED;
  // byte offsets inside one expert's weights must fit the 32-bit descriptor range
  const int64_t wbytes = ((EPI == EPI_SWIGLU) ? 2 : 1) * a.N * a.K * 2;
  if (wbytes >= (int64_t(1) << 31) || static_cast<int64_t>(BM + kFatExtraRows) * a.K * 2 >= (int64_t(1) << 31))
    return MOE_ERR_UNSUPPORTED;
  if (a.rowmap && (a.kdiv < 1 || a.a_rows * a.K * 2 >= (int64_t(1) << 31))) return MOE_ERR_UNSUPPORTED;
  hipLaunchKernelGGL((gemm_bf16_dtl_kernel<BM, BN, WM, WN, EPI, SN, BK, SP, LDS_EPI, WS>), dim3(static_cast<unsigned>(grid)),
                     dim3(64 * WM * WN), 0, st, b);
  return launch_status();
}


}  // namespace


// Expert projections: 256 token rows x 256 weight rows per tile, 8 waves
// (2 along tokens x 4 along weights, 128 x 64 each), 64-wide K stages
// loaded straight into LDS, each stage's loads spread over its 4 K slices.
moe_status gemm_bf16_gateup_swiglu(const GemmArgs& a, hipStream_t st) {
  return launch_dtl<256, 256, 2, 4, EPI_SWIGLU, 16, 64, 4, 0>(a, st);
}

// The down projection's output tile is 256 columns wide, so its epilogue
// goes through LDS (whole-row stores; measured faster on every MoE shape,
// while the 128-column SwiGLU tile of gate/up measured slower that way).
moe_status gemm_bf16_down(const GemmArgs& a, hipStream_t st) {
  return launch_dtl<256, 256, 2, 4, EPI_STORE, 16, 64, 4, 1>(a, st);
}

// Decode calls with several rows per expert (few tokens in all, weight
// streaming bound): 64-token tiles.  Gate/up keeps 256 weight rows on 4
// waves side by side; down takes 128 weight rows, so the experts' weights
// spread over twice as many tiles (32 experts of 2880 x 2880: 736 tiles
// instead of 384).  Measured at T = 32-64 against the projections' 256 x
// 256 tile: gate/up 186 -> 180 us, down 110 -> 104 us.  Down then takes two
// weight stages instead of three (48 KB of LDS, so three workgroups share a
// CU and the 736 tiles make one round instead of 1.4 rounds of two): T=64
// down 104 -> 93 us, outputs bit-identical (the K order is unchanged).
moe_status gemm_bf16_gateup_swiglu_few(const GemmArgs& a, hipStream_t st) {
  return launch_dtl<64, 256, 1, 4, EPI_SWIGLU, 16, 64, 2, 0>(a, st);
}

moe_status gemm_bf16_down_few(const GemmArgs& a, hipStream_t st) {
  return launch_dtl<64, 128, 2, 4, EPI_STORE, 16, 64, 3, 1, 2>(a, st);
}

// Router logits (many experts and tokens): the same tile kernel with an
// fp32 + bias epilogue on flat tiles of 128 experts x 64 tokens, or x 32
// tokens (4 waves) when 64-token tiles would leave CUs idle.  Measured
// against the former register-staged kernel: T=8192, E=128 24 -> 19 us;
// T=16384, E=256 100 -> 83 us; T=2048, E=256 74 -> 47 us.
moe_status gemm_bf16_logits(const GemmArgs& a, hipStream_t st) {
  if (ceil_div(a.rows, 64) * ceil_div(a.N, 128) >= 256) return launch_dtl<64, 128, 2, 4, EPI_F32B, 16, 64, 3, 0>(a, st);
  return launch_dtl<32, 128, 1, 4, EPI_F32B, 16, 64, 1, 0>(a, st);
}

}  // namespace moe
