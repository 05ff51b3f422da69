// Host replay of the MXFP4 LDS-staged kernel's loads and LDS reads (CPU
// only).
//
// The kernel's own address arithmetic -- mxl_scale_off, mxl_code_off,
// mxl_tok_off, mxl_tok_loads, mxl_code_read, mxl_tok_read, mxl_expert_row
// and mxl_scale_row, all __host__ __device__ -- is run on the host for every
// workgroup, wave, lane, load and stage of launches in several shapes, and
// builds an image of what each LDS byte holds.  Checked:
//   * every load's offset is 16-byte aligned and either wholly inside its
//     buffer's extent (the expert's codes or scales, the token rows) or past
//     it (read as zero);
//   * every 1 KB LDS destination lies inside its area (the scales, or the
//     code or token part of a stage buffer), and the areas fit the LDS the
//     kernel declares;
//   * every byte a lane reads for an MFMA holds what the arithmetic needs:
//     the scale of block b of the lane's expert row, the codes of block
//     4 jq + q of that row (inside the row), and elements 128 jq + 32 q +
//     8 m .. + 7 of token row src(m0 + i) -- the same elements of K for the
//     weights and the tokens;
//   * a skipped token load covers only rows past the expert's rows;
//   * the quads of a row cover its blocks exactly once.
// Prints the number of checks and failures; exits non-zero on a failure.
#include "decode_mx.hip"

#include <cstdio>
#include <cstdlib>
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

static bool in_or_past(long off, long extent) { return off % 16 == 0 && off >= 0 && (off >= extent || off + 16 <= extent); }

// One launch: experts with the given row counts, weights [E][brows][K/2],
// token rows gathered through a row map (entries / kdiv) when map is set.
template <bool SWIGLU>
static void replay(const char* name, int N, int K, const std::vector<int>& counts, int kdiv, bool map) {
  const int KB = K / 32, KH = K / 2, nq = KB / 4, nst = (K + 255) / 256;
  const int brows = SWIGLU ? 2 * N : N;
  const long crec = static_cast<long>(brows) * KH, srec = static_cast<long>(brows) * KB;
  std::vector<int> off(1, 0);
  for (int c : counts) off.push_back(off.back() + c);
  const int rows = off.back();
  const long trec = static_cast<long>(rows / kdiv) * K * 2;
  std::vector<int> rowmap(rows);
  for (int m = 0; m < rows; ++m) rowmap[m] = (m * 7919 + 13) % rows;   // a permutation-like map
  auto src_of = [&](int m) { return map ? clamp_off(rowmap[m], rows - 1) / kdiv : m; };
  const int CPB = SWIGLU ? 32 : 64;
  const long checks0 = g_checks;
  const int fails0 = g_fails;
  // the LDS shape the launch picks for this projection and K (the middle
  // shape of the down projection has the wide one's scale area)
  const int scb = (SWIGLU && K <= MxlNarrow::kScaleBytes / 2) ? MxlNarrow::kScaleBytes : MxlWide::kScaleBytes;
  CHECK(MxlMid::kScaleBytes == MxlWide::kScaleBytes, "middle scale area");
  CHECK(MxlWide::kLdsBytes <= 80 * 1024 && MxlMid::kLdsBytes * 3 <= 160 * 1024 && MxlNarrow::kLdsBytes <= 40 * 1024,
        "lds %d %d %d", MxlWide::kLdsBytes, MxlMid::kLdsBytes, MxlNarrow::kLdsBytes);
  CHECK(scb >= 64 * KB, "scale area for K %d", K);
  for (int cb = 0; cb * CPB < N; ++cb) {
    const int n0 = cb * CPB;
    // scales
    std::vector<long> simg(scb, -2);
    for (int w = 0; w < 4; ++w)
      for (int k = w; k * 64 < 4 * KB; k += 4) {
        CHECK((k + 1) * 1024 <= scb, "scale load %d", k);
        for (int lane = 0; lane < 64; ++lane) {
          const long o = mxl_scale_off<SWIGLU>(k * 64 + lane, n0, N, KB);
          CHECK(in_or_past(o, srec), "scale off %ld of %ld", o, srec);
          for (int b = 0; b < 16 && k * 1024 + lane * 16 + b < scb; ++b)
            simg[k * 1024 + lane * 16 + b] = o < srec ? o + b : -1;
        }
      }
    for (int rl = 0; rl < 64; ++rl)
      for (int blk = 0; blk < KB; ++blk) {
        const long want = static_cast<long>(mxl_expert_row<SWIGLU>(rl, n0, N)) * KB + blk;
        CHECK(simg[mxl_scale_row<SWIGLU>(rl) * KB + blk] == want, "%s cb %d row %d block %d", name, cb, rl, blk);
      }
    // codes, per stage
    std::vector<int> used(64 * KB, 0);
    for (int st = 0; st < nst; ++st) {
      std::vector<long> cimg(kMxlCodeBytes, -2);
      for (int w = 0; w < 4; ++w)
        for (int kk = 0; kk < 2; ++kk)
          for (int lane = 0; lane < 64; ++lane) {
            const int dst = (2 * w + kk) * 1024 + lane * 16;
            CHECK(dst + 16 <= kMxlCodeBytes, "code dst %d", dst);
            const long o = mxl_code_off<SWIGLU>(w, kk, lane, n0, N, KH) + static_cast<long>(st) * 128;
            CHECK(in_or_past(o, crec), "code off %ld of %ld", o, crec);
            CHECK(mxl_code_row(w, kk, lane) * 128 + (lane & 7) * 16 == dst, "code slot");
            for (int b = 0; b < 16; ++b) cimg[dst + b] = o < crec ? o + b : -1;
          }
      for (int w = 0; w < 4; ++w)
        for (int lane = 0; lane < 64; ++lane) {
          const int rl = 16 * w + (lane & 15), q = lane >> 4;
          for (int u = 0; u < 2; ++u) {
            const int jq = 2 * st + u;
            if (jq > nq || (jq == nq && !(KB & 3))) break;
            if (jq == nq && q >= 2) continue;          // blocks past K: zeroed by the kernel
            const int blk = 4 * jq + q;
            const int rd = mxl_code_read(rl, u, q);
            CHECK(rd >= 0 && rd + 16 <= kMxlCodeBytes, "code read %d", rd);
            CHECK(blk < KB && (blk + 1) * 16 <= KH, "block %d of %d", blk, KB);
            const long want = static_cast<long>(mxl_expert_row<SWIGLU>(rl, n0, N)) * KH + blk * 16;
            for (int b = 0; b < 16; ++b)
              CHECK(cimg[rd + b] == want + b, "%s cb %d st %d row %d q %d u %d byte %d", name, cb, st, rl, q, u, b);
            if (blk < KB) used[rl * KB + blk] += 1;
          }
        }
    }
    for (int i = 0; i < 64 * KB; ++i) CHECK(used[i] == 1, "row %d block %d used %d times", i / KB, i % KB, used[i]);
  }
  // tokens, per expert chunk and stage
  for (size_t g = 0; g + 1 < off.size(); ++g) {
    const int lo = off[g], hi = off[g + 1];
    for (int m0 = lo; m0 < hi; m0 += 16)
      for (int st = 0; st < nst; ++st) {
        std::vector<long> timg(kMxlTokBytes, -2);
        for (int w = 0; w < 4; ++w) {
          const int ntl = mxl_tok_loads(hi - m0, w);
          for (int kk = 0; kk < 2; ++kk) {
            if (kk >= ntl) {
              CHECK(m0 + 4 * w + 2 * kk >= hi, "skipped load of a present row: wave %d load %d", w, kk);
              continue;
            }
            for (int lane = 0; lane < 64; ++lane) {
              const int m = m0 + mxl_tok_row(w, kk, lane);
              const long o =
                  static_cast<long>(mxl_tok_off(m < hi ? src_of(m) : -1, K, w, kk, lane)) + static_cast<long>(st) * 512;
              CHECK(in_or_past(o, trec), "token off %ld of %ld", o, trec);
              const int dst = (2 * w + kk) * 1024 + lane * 16;
              CHECK(dst + 16 <= kMxlTokBytes, "token dst %d", dst);
              for (int b = 0; b < 16; ++b) timg[dst + b] = o < trec ? o + b : -1;
            }
          }
        }
        for (int i = 0; i < 16 && m0 + i < hi; ++i)
          for (int q = 0; q < 4; ++q)
            for (int u = 0; u < 2; ++u) {
              const int jq = 2 * st + u;
              if (jq > nq || (jq == nq && !(KB & 3))) break;
              if (jq == nq && q >= 2) continue;
              for (int m = 0; m < 4; ++m) {
                const int rd = mxl_tok_read(i, u, q, m);
                CHECK(rd >= 0 && rd + 16 <= kMxlTokBytes, "token read %d", rd);
                const long want = static_cast<long>(src_of(m0 + i)) * K * 2 + (128L * jq + 32 * q + 8 * m) * 2;
                for (int b = 0; b < 16; ++b)
                  CHECK(timg[rd + b] == want + b, "%s expert %zu m0 %d st %d row %d q %d u %d m %d", name, g, m0, st, i,
                        q, u, m);
              }
            }
      }
  }
  std::printf("%-40s checks %ld failures %d\n", name, g_checks - checks0, g_fails - fails0);
}

static std::vector<int> spread(int E, int rows, int seed) {
  std::vector<int> c(E, 0);
  unsigned x = 2463534242u + seed;
  for (int r = 0; r < rows; ++r) {
    x ^= x << 13; x ^= x >> 17; x ^= x << 5;
    c[x % E] += 1;
  }
  return c;
}

int main() {
  // gpt-oss-shaped decode (K = 2880: a half quad at the end), small shapes
  // of the parity tests, the largest K, and experts with more than 16 rows
  replay<true>("gate/up d2880 f2880 T64 k4", 2880, 2880, spread(32, 256, 1), 4, true);
  replay<false>("down d2880 f2880 T64", 2880, 2880, spread(32, 256, 1), 1, false);
  replay<true>("gate/up d576 f640 T37 k4", 640, 576, spread(32, 148, 2), 4, true);
  replay<false>("down d576 f640 T37", 576, 640, spread(32, 148, 2), 1, false);
  replay<true>("gate/up K2048 N192", 192, 2048, spread(16, 40, 3), 1, false);
  replay<false>("down K8192 N64", 64, 8192, spread(8, 200, 4), 1, false);
  replay<true>("gate/up K8192 N64 (>16 rows)", 64, 8192, {40, 0, 33, 17, 1, 0, 9, 100}, 1, false);
  replay<true>("gate/up K64 N64", 64, 64, spread(4, 20, 5), 2, true);
  replay<false>("down K64 N192", 192, 64, spread(4, 20, 5), 1, false);
  std::printf("total checks %ld failures %d\n", g_checks, g_fails);
  return g_fails ? 1 : 0;
}
