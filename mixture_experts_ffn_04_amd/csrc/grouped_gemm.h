// Grouped GEMM machinery for the MoE layer on gfx950.
//
// One launch computes, for every group g (an expert) owning the rows
// [off[g], off[g+1]) of A:
//
//     C[r][n] = sum_k A[r][k] * B[g][n][k]          (B row-major [N][K])
//
// A and B are both K-contiguous, so every MFMA operand is a 16-byte run of
// one row.  The epilogue is fused:
//   EPI_STORE   C in the element type                 (down projection)
//   EPI_SWIGLU  B's rows [0, N) are gate and [N, 2N) are up; output column n
//               is silu(C_gate[n]) * C_up[n]          (gate/up projection)
//   EPI_F32B    C + bias[n] as fp32                   (router logits)
//
// This is the "grouped_mm" expert execution of the article "Mixture of
// Experts (MoEs) in Transformers" (section "Expert Backend"): the token rows
// are already sorted by expert and one grouped GEMM covers all experts.
//
// Tile schedule.  Each workgroup reads offsets[] (G <= 256 entries) and scans
// the per-group tile counts itself, so there is no host round trip, no
// workspace, and empty experts cost nothing.  Tiles are numbered group-major,
// then in blocks of SN column tiles, then by row tile, then by the column
// tile inside the block, so the workgroups that run together share their
// weight tiles (same column block) and their token tiles (same row tile).
// Workgroup ids are remapped so that even ids walk the first half of that
// order and odd ids the second.  (Measured on the MoE shapes against no
// remap and against 4- and 8-way remaps -- one contiguous stretch per XCD
// -- and column blocks of 2 to 16: two halves with 16-wide blocks was the
// fastest, by 2-11% over one stretch per XCD, although it fetches more
// from beyond L2.)
//
// Row tiles.  A group's rows are dealt to its row tiles in whole 32-row
// fragments, as evenly as possible (row_tiles, tile_coords).  The rows per
// row tile are BM, or BM with a group's small last remainder folded into its
// other tiles (fat tiles, where the launcher allows them), or -- in a
// launch of only a few rounds of tiles -- a per-launch choice that every
// workgroup makes identically from the offsets (tile_rows_for).  Which rows
// a tile holds never changes a result: each output keeps its K order.
#pragma once

#include "common.h"

namespace moe {

enum { EPI_STORE = 0, EPI_SWIGLU = 1, EPI_F32B = 2 };

struct GemmArgs {
  const void* A;          // [rows][K]
  const void* B;          // [G][b_rows][K], b_rows = N (2N for SWIGLU)
  const int32_t* off;     // [G+1] group row offsets (device); NULL -> one group [0, rows)
  const float* bias;      // [N] for EPI_F32B (may be NULL)
  void* C;                // [rows][N] (SWIGLU: [rows][N] too, N = f)
  int64_t rows;           // rows of A and C
  int64_t K;
  int64_t N;              // output columns
  int G;                  // groups
  // Optional row gather (bf16 tile kernel): A row r is A[rowmap[r] / kdiv]
  // (rowmap entries clamped to [0, rows)); A then has a_rows rows.
  const int32_t* rowmap;
  int kdiv;
  int64_t a_rows;
  // Set by the launcher, not by callers: the launch is short enough (fewer
  // than kAdaptRounds rounds of full row tiles) for the tile rows to be
  // chosen per launch, and its grid covers the smallest choice.
  int adapt_rows;
  // Set by the launcher, not by callers: fat tiles are allowed, where a
  // group's last remainder of at most kFatExtraRows rows is shared out over
  // its other row tiles, which then hold up to BM + kFatExtraRows rows.
  int fat_rows;
  // Set by the launcher, not by callers: slots walk the tile order in 4
  // interleaved quarters instead of 2 halves (tile_order).
  int quarters;
};

constexpr int kComputeUnits = 256;   // MI355X: compute units, one tile workgroup each
constexpr int kAdaptRounds = 4;
constexpr int kRowChoices = 4;       // BM, BM - 32, BM - 64, BM - 96 rows per row tile
constexpr int kFatExtraRows = 64;

struct TileLoc {
  int g;         // group
  int row0;      // first A/C row of the tile
  int row_end;   // end of the tile's rows (inside its group)
  int n0;        // first output column
};

// Row tiles of a group of r rows at tr rows per tile.  tr > BM means fat
// tiles: BM-row tiles, with a last remainder of at most tr - BM rows shared
// out over the group's other row tiles instead of taking a tile of its own.
template <int BM>
__host__ __device__ __forceinline__ int row_tiles(int r, int tr) {
  if (tr <= BM) return (r + tr - 1) / tr;
  int m = (r + BM - 1) / BM;
  if (m > 1 && r - (m - 1) * BM <= tr - BM) --m;
  return m;
}

// Rows per row tile (a value above BM means fat tiles, see row_tiles).
// Without a.adapt_rows: BM, or fat tiles where the launcher allows them.  A
// launch of a few rounds of tiles leaves most CUs idle in its last round,
// so with a.adapt_rows set every workgroup picks, from the same offsets and
// so identically, among BM, BM - 32, BM - 64, BM - 96 rows and (where
// allowed) fat tiles, the choice that minimises (rounds of tiles) x (32-row
// fragments of the largest tile), ties to fat tiles, then to more rows.
// Measured on 8 experts of ~1024 rows, K = 14336, N = 4096: 192 rows (752
// tiles, 2.9 rounds) ran 5% faster than 256 rows (592 tiles, 2.3 rounds),
// and fat tiles (512 tiles, 2 rounds) 2% faster again; launches of more
// rounds measured fastest with 256-row (or fat) tiles.  Contains one
// workgroup barrier.  s_red: kRowReduce * NT/64 ints of LDS.
constexpr int kRowReduce = kRowChoices + 3;
template <int NT, int BM, int BNO>
__device__ __forceinline__ int tile_rows_for(const GemmArgs& a, int r, int ntiles, int* s_red) {
  constexpr int FAT = BM + kFatExtraRows;
  if (BM < 32 * kRowChoices || !a.adapt_rows) return a.fat_rows ? FAT : BM;
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  // per candidate tile counts; then the largest group's rows, the fat tile
  // count and the fragments of the largest fat-mode tile
  int v[kRowReduce];
#pragma unroll
  for (int c = 0; c < kRowChoices; ++c) v[c] = ((r + BM - 32 * c - 1) / (BM - 32 * c)) * ntiles;
  v[kRowChoices] = r;
  const int mf = r > 0 ? row_tiles<BM>(r, FAT) : 1;
  v[kRowChoices + 1] = r > 0 ? mf * ntiles : 0;
  v[kRowChoices + 2] = ((r + 31) / 32 + mf - 1) / mf;
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) {
#pragma unroll
    for (int c = 0; c < kRowReduce; ++c) {
      const int u = __shfl_xor(v[c], o, 64);
      v[c] = (c == kRowChoices || c == kRowChoices + 2) ? max(v[c], u) : v[c] + u;
    }
  }
  if (lane == 0) {
#pragma unroll
    for (int c = 0; c < kRowReduce; ++c) s_red[c * (NT / 64) + w] = v[c];
  }
  __syncthreads();
  int tot[kRowReduce];
#pragma unroll
  for (int c = 0; c < kRowReduce; ++c) {
    tot[c] = 0;
#pragma unroll
    for (int i = 0; i < NT / 64; ++i) {
      const int u = s_red[c * (NT / 64) + i];
      tot[c] = (c == kRowChoices || c == kRowChoices + 2) ? max(tot[c], u) : tot[c] + u;
    }
  }
  const int maxf = (tot[kRowChoices] + 31) / 32;       // fragments of the largest group
  int best = BM, best_cost = 0x7fffffff;
  if (a.fat_rows) {
    best = FAT;
    best_cost = ((tot[kRowChoices + 1] + kComputeUnits - 1) / kComputeUnits) * tot[kRowChoices + 2];
  }
#pragma unroll
  for (int c = 0; c < kRowChoices; ++c) {
    const int rows_c = BM - 32 * c;
    const int cost = ((tot[c] + kComputeUnits - 1) / kComputeUnits) * min(rows_c / 32, maxf);
    if (cost < best_cost) {
      best_cost = cost;
      best = rows_c;
    }
  }
  return best;
}

// Tile counts of the groups and their exclusive scan, for all NT threads:
// thread t < G gets its group's row range [lo, hi), tile count cnt and the
// index excl of its first tile; every thread gets the total and the rows
// per row tile tr.  Contains one or two workgroup barriers.
// s_wsum: NT/64 ints of LDS; s_red as for tile_rows_for.
template <int NT, int BM, int BNO>
__device__ __forceinline__ int scan_tiles(const GemmArgs& a, int& lo, int& hi, int& cnt, int& excl, int& tr,
                                          int* s_wsum, int* s_red) {
  static_assert(NT >= kMaxE, "one group per thread");
  const int t = threadIdx.x;
  const int rows = static_cast<int>(a.rows);
  const int ntiles = static_cast<int>((a.N + BNO - 1) / BNO);
  lo = 0;
  hi = 0;
  cnt = 0;
  if (t < a.G) {
    lo = a.off ? clamp_off(a.off[t], rows) : 0;
    hi = a.off ? clamp_off(a.off[t + 1], rows) : rows;
    if (hi < lo) hi = lo;
  }
  tr = tile_rows_for<NT, BM, BNO>(a, hi - lo, ntiles, s_red);
  cnt = row_tiles<BM>(hi - lo, tr) * ntiles;
  const int lane = t & 63, w = t >> 6;
  int v = cnt;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    int u = __shfl_up(v, o, 64);
    if (lane >= o) v += u;
  }
  if (lane == 63) s_wsum[w] = v;
  __syncthreads();
  int base = 0, total = 0;
#pragma unroll
  for (int i = 0; i < NT / 64; ++i) {
    int s = s_wsum[i];
    base += (i < w) ? s : 0;
    total += s;
  }
  excl = base + v - cnt;
  return total;
}

// Logical tile index of launch slot bid.  Even slots walk the first half of
// the order, odd slots the second, so the tiles running together on one XCD
// (slots are dealt to the 8 XCDs round-robin) come from a stretch of the
// order shared with three other XCDs: fewer experts' weights are in flight
// at once than with one contiguous stretch per XCD.
// With quarters, slot s walks quarter s mod 4 instead (short K loops).
__device__ __forceinline__ int tile_order(int bid, int total, bool quarters) {
  if (quarters) {
    const int q = total >> 2;
    return (bid < (q << 2)) ? ((bid & 3) * q + (bid >> 2)) : bid;
  }
  const int q = total >> 1;
  return (bid < (q << 1)) ? ((bid & 1) * q + (bid >> 1)) : bid;
}

// Rows [row0, row_end) of row tile mt of a group with rows [glo, ghi) cut
// into mt_g row tiles: the group's 32-row fragments are dealt as evenly as
// possible over its row tiles (the first F % mt_g take one more), so no
// tile of a ragged group is left with a sliver of rows that still streams a
// whole weight tile.
__host__ __device__ __forceinline__ void tile_rows(int glo, int ghi, int mt, int mt_g, int& row0, int& row_end) {
  const int nf = (ghi - glo + 31) / 32;
  const int fq = nf / mt_g, fr = nf - fq * mt_g;
  const int f0 = mt * fq + (mt < fr ? mt : fr);
  const int f1 = f0 + fq + (mt < fr ? 1 : 0);
  row0 = glo + 32 * f0;
  row_end = ghi < glo + 32 * f1 ? ghi : glo + 32 * f1;
}

// Tile coordinates of logical tile `local` of group g (rows [glo, ghi)):
// column blocks of SN tiles, row tiles within a block, a narrower last block
// when SN does not divide the column tiles.
template <int BM, int BNO, int SN>
__device__ __forceinline__ TileLoc tile_coords(const GemmArgs& a, int g, int glo, int ghi, int local, int tr) {
  const int ntiles = static_cast<int>((a.N + BNO - 1) / BNO);
  const int mt_g = row_tiles<BM>(ghi - glo, tr);
  const int nbf = ntiles / SN;
  int mt, nt;
  if (local < nbf * mt_g * SN) {
    const int nb = local / (mt_g * SN);
    const int r = local - nb * (mt_g * SN);
    mt = r / SN;
    nt = nb * SN + (r - mt * SN);
  } else {
    const int snr = ntiles - nbf * SN;
    const int r = local - nbf * mt_g * SN;
    mt = r / snr;
    nt = nbf * SN + (r - mt * snr);
  }
  int row0, row_end;
  tile_rows(glo, ghi, mt, mt_g, row0, row_end);
  // workgroup-uniform: keep them in scalar registers
  TileLoc tl;
  tl.g = __builtin_amdgcn_readfirstlane(g);
  tl.row0 = __builtin_amdgcn_readfirstlane(row0);
  tl.row_end = __builtin_amdgcn_readfirstlane(row_end);
  tl.n0 = __builtin_amdgcn_readfirstlane(nt * BNO);
  return tl;
}

// LDS scratch of locate_tile, in ints.
constexpr int locate_scratch_ints(int NT) { return NT / 64 * (kRowReduce + 1) + 4; }

// Locate this workgroup's tile.  Must be called by all NT threads; returns
// false (for the whole workgroup) when the block id is past the last tile.
//   BM     rows per tile, BNO output columns per tile, SN column-block width
//   scratch  locate_scratch_ints(NT) ints of LDS, free again once this
//            returns and every thread has passed one more workgroup barrier
template <int NT, int BM, int BNO, int SN>
__device__ __forceinline__ bool locate_tile(const GemmArgs& a, TileLoc& tl, int* scratch) {
  int* s_red = scratch + NT / 64;
  int* s_hit = s_red + NT / 64 * kRowReduce;
  int lo, hi, cnt, excl, tr;
  const int total = scan_tiles<NT, BM, BNO>(a, lo, hi, cnt, excl, tr, scratch, s_red);
  const int bid = static_cast<int>(blockIdx.x);
  if (bid >= total) return false;     // uniform: total is the same in every thread
  const int L = tile_order(bid, total, a.quarters != 0);
  if (static_cast<int>(threadIdx.x) < a.G && cnt > 0 && L >= excl && L < excl + cnt) {
    s_hit[0] = threadIdx.x;
    s_hit[1] = lo;
    s_hit[2] = hi;
    s_hit[3] = excl;
  }
  __syncthreads();
  tl = tile_coords<BM, BNO, SN>(a, s_hit[0], s_hit[1], s_hit[2], L - s_hit[3], tr);
  return true;
}

// The same with scratch of its own.
template <int NT, int BM, int BNO, int SN>
__device__ __forceinline__ bool locate_tile(const GemmArgs& a, TileLoc& tl) {
  __shared__ int scratch[locate_scratch_ints(NT)];
  return locate_tile<NT, BM, BNO, SN>(a, tl, scratch);
}

// Upper bound on the tiles of a grouped launch (used as the grid size):
// every group adds at most one partial row tile.
inline int64_t grouped_tile_bound(int64_t rows, int G, int BM, int64_t N, int BNO) {
  return (ceil_div(rows, BM) + G) * ceil_div(N, BNO);
}

}  // namespace moe
