// Host replay of the bf16 tile kernel's direct-to-LDS loads (CPU only).
//
// The kernel's own address arithmetic -- DtlShape, tile_rows, row_tiles,
// tile_buffers and dma_offsets, all __host__ __device__ -- is run on the
// host for every tile, wave, lane and load instruction of launches in each
// shipped tile shape, and every buffer load is checked against what it is
// allowed to touch:
//   * a descriptor's extent (num_records) never reaches past its
//     allocation: expert g's weights, or the token rows;
//   * a lane whose offset is inside the extent (the hardware then loads it)
//     reads 16 bytes of the row it means, even at the last K stage: the
//     stage's K offset travels in the scalar offset, which the hardware
//     range check does not include;
//   * every valid token / weight row of the tile is loaded, and a row past
//     the tile's rows or past N is either outside the extent (read as zero)
//     or, for a gathered token row, row 0 of the tokens;
//   * each instruction's 1 KB LDS destination lies inside its stage buffer
//     and the stages fit the LDS the kernel declares.
// Prints the number of checks and failures; exits non-zero on a failure.
#include "gemm_bf16.hip"

#include <cstdio>
#include <cstdlib>
#include <cmath>
#include <vector>

using namespace moe;

static long g_checks = 0;
static int g_fails = 0;

#define CHECK(cond, ...)                      \
  do {                                        \
    ++g_checks;                               \
    if (!(cond)) {                            \
      if (g_fails++ < 20) {                   \
        std::printf("FAIL %s: ", #cond);      \
        std::printf(__VA_ARGS__);             \
        std::printf("\n");                    \
      }                                       \
    }                                         \
  } while (0)

template <int BM, int BN, int WM, int WN, int EPI, int WS = 3>
void replay(const char* name, const std::vector<int>& in_counts, int64_t K, int64_t N, int kdiv,
            const std::vector<int>& row_choices) {
  typedef DtlShape<BM, BN, WM, WN, EPI, 64, WS> S;
  constexpr int CH = S::CH, RPI = S::RPI, NW = S::NW;
  static_assert(S::LDS_UNITS * 16 <= 160 * 1024, "LDS");
  // two weight stages: three workgroups share a CU
  static_assert(WS == 3 || 3 * S::LDS_UNITS * 16 <= 160 * 1024, "LDS of three workgroups");
  static_assert(!S::FAT_OK || 2 * S::WSTG + 2 * S::XSTGF <= S::LDS_UNITS, "fat stages");
  const bool gather = kdiv > 0;
  std::vector<int> counts_v(in_counts);
  const int G = static_cast<int>(counts_v.size());
  if (gather) {
    // the gathered calls take rows = T * k routed rows (the entry points
    // reject rows % k != 0): pad the last group
    int total = 0;
    for (int c : counts_v) total += c;
    counts_v[G - 1] += (kdiv - total % kdiv) % kdiv;
  }
  const std::vector<int>& counts = counts_v;
  std::vector<int> off(G + 1, 0);
  for (int g = 0; g < G; ++g) off[g + 1] = off[g] + counts[g];
  const int64_t rows = off[G];
  // a row map as the sort writes it: a permutation of the routed pairs
  std::vector<int32_t> rowmap(rows);
  for (int64_t r = 0; r < rows; ++r) rowmap[r] = static_cast<int32_t>((r * 7919 + 13) % rows);
  if (gather) {
    std::vector<char> seen(rows, 0);
    bool perm = true;
    for (int64_t r = 0; r < rows; ++r) perm = perm && !seen[rowmap[r]]++;
    if (!perm)
      for (int64_t r = 0; r < rows; ++r) rowmap[r] = static_cast<int32_t>(rows - 1 - r);
  }
  GemmArgs a{};
  a.off = nullptr;
  a.rows = rows;
  a.K = K;
  a.N = N;
  a.G = G;
  a.rowmap = gather ? rowmap.data() : nullptr;
  a.kdiv = gather ? kdiv : 1;
  a.a_rows = gather ? rows / kdiv : rows;
  const int64_t rowb = K * 2;
  const int64_t a_bytes = a.a_rows * rowb;
  const int64_t brows = EPI == EPI_SWIGLU ? 2 * N : N;
  const int64_t b_bytes = G * brows * rowb;
  const int64_t soff_max = (K / 64 - 1) * 128;         // the last stage's K offset
  const int ntiles = static_cast<int>((N + S::BNO - 1) / S::BNO);
  long tiles = 0;
  for (int tr : row_choices) {
    for (int g = 0; g < G; ++g) {
      const int r = counts[g];
      if (r == 0) continue;
      const int mt_g = row_tiles<BM>(r, tr);
      for (int mt = 0; mt < mt_g; ++mt) {
        int row0, row_end;
        tile_rows(off[g], off[g + 1], mt, mt_g, row0, row_end);
        for (int nt = 0; nt < ntiles; ++nt) {
          ++tiles;
          TileLoc tl{g, row0, row_end, nt * S::BNO};
          const TileBuffers tb = tile_buffers<EPI, BM, S::FAT_OK, S::BMF>(a, tl);
          const bool fat = S::FAT_OK && tb.vrows > BM;
          CHECK(tb.vrows >= 1 && tb.vrows <= (fat ? S::BMF : BM), "%s g=%d tile rows %d", name, g, tb.vrows);
          CHECK(tb.wbase >= 0 && tb.wbase + tb.wrecords <= b_bytes && tb.wbase + tb.wrecords <= (g + 1) * brows * rowb,
                "%s g=%d weight extent", name, g);
          CHECK(tb.abase >= 0 && tb.abase + tb.arecords <= a_bytes, "%s g=%d token extent", name, g);
          const int NX = fat ? S::LXF : S::LX;
          const int NL = fat ? S::LPF : S::LPS;
          const int tm = fat ? S::TMF : S::TM;
          const int xstage = (fat ? S::XSTGF : S::XSTG) * 16;
          for (int wave = 0; wave < NW; ++wave) {
            const int wm = wave / WN, wn = wave % WN;
            for (int lane = 0; lane < 64; ++lane) {
              int voff[S::LPF > S::LPS ? S::LPF : S::LPS], dst[S::LPF > S::LPS ? S::LPF : S::LPS];
              if (fat) {
                int v[S::LPF], d[S::LPF];
                dma_offsets<EPI, BN, CH, RPI, NW, WN, S::LXF, S::LPF>(a, tl, rowb, gather, wave, wm, wn, lane, tm,
                                                                      v, d);
                for (int i = 0; i < S::LPF; ++i) voff[i] = v[i], dst[i] = d[i];
              } else {
                int v[S::LPS], d[S::LPS];
                dma_offsets<EPI, BN, CH, RPI, NW, WN, S::LX, S::LPS>(a, tl, rowb, gather, wave, wm, wn, lane, tm, v,
                                                                     d);
                for (int i = 0; i < S::LPS; ++i) voff[i] = v[i], dst[i] = d[i];
              }
              for (int i = 0; i < NL; ++i) {
                const bool tok = i < NX;
                const int stage = tok ? xstage : S::WSTG * 16;
                CHECK(dst[i] >= 0 && dst[i] + 1024 <= stage, "%s LDS dst %d stage %d", name, dst[i], stage);
                const int trow = dst[i] / (CH * 16) + lane / CH;      // the tile row this lane loads
                CHECK(voff[i] >= 0, "%s negative offset", name);
                const int64_t base = tok ? tb.abase : tb.wbase;
                const int64_t recs = tok ? tb.arecords : tb.wrecords;
                const int64_t alloc = tok ? a_bytes : b_bytes;
                const bool loaded = voff[i] < recs;
                if (loaded) {
                  CHECK(base + voff[i] + soff_max + 16 <= alloc, "%s %s load past the allocation", name,
                        tok ? "token" : "weight");
                  CHECK(voff[i] % rowb + soff_max + 16 <= rowb, "%s load crosses into the next row", name);
                }
                if (tok) {
                  if (trow < tb.vrows) {
                    CHECK(loaded, "%s valid token row %d not loaded", name, trow);
                    const int64_t want = gather ? clamp_off(rowmap[row0 + trow], static_cast<int>(rows) - 1) / kdiv
                                                : trow;
                    CHECK(voff[i] / rowb == want, "%s token row %d reads row %lld", name, trow,
                          static_cast<long long>(voff[i] / rowb));
                  } else if (!gather) {
                    CHECK(!loaded, "%s token row %d past the tile is loaded", name, trow);
                  } else {
                    CHECK(voff[i] / rowb == 0, "%s gathered row past the tile reads row %lld", name,
                          static_cast<long long>(voff[i] / rowb));
                  }
                } else {
                  int64_t col, grow;                 // output column and weight row within expert g
                  if (EPI == EPI_SWIGLU) {
                    const int half = trow / (BN / 2);
                    col = tl.n0 + trow - half * (BN / 2);
                    grow = half * N + col;
                  } else {
                    col = tl.n0 + trow;
                    grow = trow;                      // relative to the tile's first column
                  }
                  if (col < N) {
                    CHECK(loaded && voff[i] / rowb == grow, "%s weight row %d", name, trow);
                  } else if (EPI != EPI_SWIGLU || grow >= 2 * N) {
                    // past the last output column: outside the extent, read as zero
                    CHECK(!loaded, "%s weight row past N is loaded", name);
                  }
                  // (a gate row past N reads one of the expert's up rows, inside
                  // the extent checked above; its column is never stored)
                }
              }
            }
          }
        }
      }
    }
  }
  std::printf("%-34s tiles %8ld\n", name, tiles);
}

static std::vector<int> zipf_counts(int E, int rows, double s, int seed) {
  // a skewed load with empty experts, like the Zipf-biased workloads
  std::vector<int> c(E, 0);
  std::vector<double> p(E);
  double z = 0;
  for (int e = 0; e < E; ++e) z += (p[e] = 1.0 / std::pow(e + 1.0, s));
  unsigned x = 2463534242u + seed;
  for (int i = 0; i < rows; ++i) {
    x ^= x << 13, x ^= x >> 17, x ^= x << 5;
    double u = (x % 1000003) / 1000003.0 * z;
    int e = 0;
    while (e < E - 1 && (u -= p[e]) > 0) ++e;
    ++c[(e * 37 + seed) % E];
  }
  c[(E - 1 + seed) % E] = 0;
  return c;
}

int main() {
  const std::vector<int> all_rows = {256, 224, 192, 160, 320};
  const std::vector<int> ragged = {967, 1000, 1088, 1072, 1030, 300, 530, 256, 100, 31, 0, 1};
  // expert projections, 256 x 256 tiles (and fat tiles), plain and gathered
  replay<256, 256, 2, 4, EPI_SWIGLU>("gate/up 256x256 K4096 N14336", ragged, 4096, 14336, 0, all_rows);
  replay<256, 256, 2, 4, EPI_SWIGLU>("gate/up 256x256 gather k2", ragged, 4096, 576, 2, all_rows);
  replay<256, 256, 2, 4, EPI_SWIGLU>("gate/up 256x256 Zipf K7168 N2048", zipf_counts(256, 16384, 1.0, 5), 7168, 2048,
                                     8, {256, 320});
  replay<256, 256, 2, 4, EPI_SWIGLU>("gate/up 256x256 Zipf K2048 N768", zipf_counts(128, 8192, 1.1, 4), 2048, 768, 8,
                                     {256});
  replay<256, 256, 2, 4, EPI_STORE>("down 256x256 K14336 N4096", ragged, 14336, 4096, 0, all_rows);
  replay<256, 256, 2, 4, EPI_STORE>("down 256x256 N1088 (ragged columns)", ragged, 4096, 1088, 0, all_rows);
  replay<256, 256, 2, 4, EPI_STORE>("down 256x256 Zipf K2048 N7168", zipf_counts(256, 16384, 1.0, 7), 2048, 7168, 0,
                                    {256});
  replay<256, 256, 2, 4, EPI_STORE>("down 256x256 K64 (one stage)", ragged, 64, 320, 0, all_rows);
  // decode-sized tiles
  replay<64, 256, 1, 4, EPI_SWIGLU>("gate/up 64x256 K2880 N2880", zipf_counts(32, 256, 0.5, 1), 2880, 2880, 0,
                                    {64});
  replay<64, 256, 1, 4, EPI_SWIGLU>("gate/up 64x256 gather k4", zipf_counts(32, 256, 0.5, 2), 2880, 2880, 4, {64});
  replay<64, 128, 2, 4, EPI_STORE>("down 64x128 K2880 N2880", zipf_counts(32, 256, 0.5, 3), 2880, 2880, 0, {64});
  replay<64, 128, 2, 4, EPI_STORE, 2>("down 64x128 two stages K2880 N2880", zipf_counts(32, 256, 0.5, 3), 2880, 2880,
                                      0, {64});
  replay<64, 128, 2, 4, EPI_STORE, 2>("down 64x128 two stages K64 (one stage)", {8, 9, 0, 12}, 64, 320, 0, {64});
  // router logits on flat tiles (one group of T rows, N = experts)
  replay<64, 128, 2, 4, EPI_F32B>("logits 64x128 K7168 N256", {16384}, 7168, 256, 0, {64});
  replay<32, 128, 1, 4, EPI_STORE>("down 32x128 K2880 N2880", {8, 9, 7, 12, 0, 8, 31, 1}, 2880, 2880, 0, {32});
  replay<64, 128, 1, 4, EPI_STORE>("down 64x128w4 K2880 N2880", {8, 9, 7, 12, 0, 8, 31, 1}, 2880, 2880, 0, {64});
  replay<64, 256, 1, 4, EPI_STORE>("down 64x256 K2880 N2880", {8, 9, 7, 12, 0, 8, 31, 1}, 2880, 2880, 0, {64});
  replay<128, 128, 2, 4, EPI_F32B>("logits 128x128 K7168 N256", {16384}, 7168, 256, 0, {128});
  replay<128, 128, 2, 4, EPI_F32B>("logits 128x128 K64 N200 (ragged)", {300}, 64, 200, 0, {128});
  replay<64, 256, 2, 4, EPI_F32B>("logits 64x256 K7168 N256", {16384}, 7168, 256, 0, {64});
  replay<64, 256, 2, 4, EPI_F32B>("logits 64x256 K64 N200 (ragged)", {300}, 64, 200, 0, {64});
  replay<32, 256, 1, 4, EPI_F32B>("logits 32x256 K7168 N256", {16384}, 7168, 256, 0, {32});
  replay<32, 256, 1, 4, EPI_F32B>("logits 32x256 K64 N200 (ragged)", {300}, 64, 200, 0, {32});
  replay<32, 128, 1, 4, EPI_F32B>("logits 32x128 K2048 N128", {8192}, 2048, 128, 0, {32});
  replay<64, 128, 2, 4, EPI_F32B>("logits 64x128 K64 N40 (ragged)", {300}, 64, 40, 0, {64});
  std::printf("checks %ld failures %d\n", g_checks, g_fails);
  return g_fails ? 1 : 0;
}
