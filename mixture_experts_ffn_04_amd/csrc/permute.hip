// Order the routed (token, slot) pairs by expert ID so each expert's pairs
// are contiguous -- the first step of the "grouped_mm" strategy (article
// "Mixture of Experts (MoEs) in Transformers", section "Expert Backend") --
// and gather the token rows into that order.
//
// Four launches (two when all pairs fit one chunk: histogram, scan and
// scatter then share one workgroup), no host synchronisation:
//   1. histogram  chunks of kChunk pairs; per-chunk expert counts with LDS
//                 atomics (order-free, so deterministic) -> ws counts[chunk][E]
//   2. scan       one workgroup: per expert, running sum over chunks (the
//                 chunk's base inside the expert's group), then an exclusive
//                 scan over experts -> counts, offsets, per-chunk bases
//   3. scatter    four waves per chunk, each walking a quarter of its pairs
//                 64 at a time in order from its own base (the chunk's base
//                 plus the counts of the waves before it); the rank of a pair
//                 among equal experts in the wave comes from ballots on the
//                 bits of the expert id (a match-any), so positions are
//                 stable without atomics on the ranks
//   4. gather     x_perm[r] = x[perm[r] / k], 16-byte loads and stores, one
//                 wave per row
#include <mutex>

#include "common.h"

namespace moe {
namespace {

constexpr int kChunk = 1024;   // pairs per chunk
constexpr int kScanBatch = 16; // chunks loaded together by the scan

size_t ws_bytes_for(int64_t P, int E) {
  const int64_t chunks = ceil_div(P, kChunk);
  return static_cast<size_t>(chunks) * static_cast<size_t>(E) * sizeof(int32_t);
}

__global__ __launch_bounds__(256) void hist_kernel(const int32_t* __restrict__ ids, int P, int E,
                                                   int32_t* __restrict__ cc) {
  __shared__ int h[kMaxE];
  for (int e = threadIdx.x; e < E; e += 256) h[e] = 0;
  __syncthreads();
  const int p0 = blockIdx.x * kChunk;
  const int p1 = min(P, p0 + kChunk);
  for (int p = p0 + threadIdx.x; p < p1; p += 256) {
    const int e = ids[p];
    if (e >= 0 && e < E) atomicAdd(&h[e], 1);
  }
  __syncthreads();
  for (int e = threadIdx.x; e < E; e += 256) cc[static_cast<int64_t>(blockIdx.x) * E + e] = h[e];
}

// One workgroup of kScanParts x 256 threads (E <= 256): thread (part, e)
// owns expert e's counts in chunks [part*cq, (part+1)*cq), so each thread
// walks a quarter of the chunks.  Pass 1 sums its chunks; the part sums
// give each thread its base inside the expert's group, and an exclusive
// scan over the experts' totals gives offsets; pass 2 rewrites every
// chunk's count as that chunk's first row.  Loads of kScanBatch chunks are
// issued together (one memory round trip per batch).
constexpr int kScanParts = 4;

__global__ __launch_bounds__(256 * kScanParts) void scan_kernel(int32_t* __restrict__ cc, int chunks, int E,
                                                                int32_t* __restrict__ counts,
                                                                int32_t* __restrict__ offsets) {
  __shared__ int psum[kScanParts][kMaxE];
  __shared__ int eoff[kMaxE];
  __shared__ int wsum[4];
  const int e = threadIdx.x & (kMaxE - 1);
  const int part = threadIdx.x / kMaxE;
  const int cq = (chunks + kScanParts - 1) / kScanParts;
  const int c_lo = min(chunks, part * cq), c_hi = min(chunks, c_lo + cq);
  int mine = 0;
  if (e < E) {
    for (int c0 = c_lo; c0 < c_hi; c0 += kScanBatch) {
      int v[kScanBatch];
#pragma unroll
      for (int j = 0; j < kScanBatch; ++j) v[j] = c0 + j < c_hi ? cc[static_cast<int64_t>(c0 + j) * E + e] : 0;
#pragma unroll
      for (int j = 0; j < kScanBatch; ++j) mine += v[j];
    }
  }
  psum[part][e] = mine;
  __syncthreads();
  int before = 0, tot = 0;
#pragma unroll
  for (int q = 0; q < kScanParts; ++q) {
    before += q < part ? psum[q][e] : 0;
    tot += psum[q][e];
  }
  // exclusive scan of the experts' totals, held by the first 256 threads
  // (every thread takes part in the barriers)
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  int v = (part == 0 && e < E) ? tot : 0;
  const int c = v;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int u = __shfl_up(v, o, 64);
    if (lane >= o) v += u;
  }
  if (part == 0 && lane == 63) wsum[w] = v;
  __syncthreads();
  if (part == 0) {
    int base = 0;
    for (int i = 0; i < w; ++i) base += wsum[i];
    const int excl = base + v - c;
    if (e < E) {
      counts[e] = tot;
      offsets[e] = excl;
      eoff[e] = excl;
    }
    if (e == E - 1) offsets[E] = excl + tot;
  }
  __syncthreads();
  if (e < E) {
    int run = eoff[e] + before;
    for (int c0 = c_lo; c0 < c_hi; c0 += kScanBatch) {
      int v[kScanBatch];
#pragma unroll
      for (int j = 0; j < kScanBatch; ++j) v[j] = c0 + j < c_hi ? cc[static_cast<int64_t>(c0 + j) * E + e] : 0;
#pragma unroll
      for (int j = 0; j < kScanBatch; ++j) {
        if (c0 + j < c_hi) cc[static_cast<int64_t>(c0 + j) * E + e] = run;   // first row of the chunk in e's group
        run += v[j];
      }
    }
  }
}

// One workgroup of 4 waves per chunk; wave w takes the chunk's pairs
// [256w, 256w + 256).  The waves first count their pairs per expert (LDS
// atomics, order-free), thread e then turns the chunk's base in expert e's
// group into one base per wave (the counts of the waves before it added),
// and each wave walks its pairs 64 at a time in order.  Its ids are all
// loaded before the walk.
constexpr int kScatterWaves = 4;
constexpr int kScatterSteps = kChunk / (64 * kScatterWaves);

__global__ __launch_bounds__(64 * kScatterWaves) void scatter_kernel(const int32_t* __restrict__ ids, int P, int E,
                                                                     int nbits, const int32_t* __restrict__ cc,
                                                                     int32_t* __restrict__ perm,
                                                                     int32_t* __restrict__ inv_perm) {
  __shared__ int cnt[kScatterWaves][kMaxE];
  __shared__ int base[kScatterWaves][kMaxE];
  const int t = threadIdx.x, lane = t & 63, w = t >> 6;
  const int p0 = blockIdx.x * kChunk + w * (64 * kScatterSteps);
  const int pend = min(P, blockIdx.x * kChunk + kChunk);
  int idv[kScatterSteps];
#pragma unroll
  for (int i = 0; i < kScatterSteps; ++i) {
    const int p = p0 + 64 * i + lane;
    idv[i] = p < pend ? ids[p] : -1;
  }
  for (int e = lane; e < E; e += 64) cnt[w][e] = 0;
  __syncthreads();
#pragma unroll
  for (int i = 0; i < kScatterSteps; ++i)
    if (idv[i] >= 0 && idv[i] < E) atomicAdd(&cnt[w][idv[i]], 1);
  __syncthreads();
  if (t < E) {
    int b = cc[static_cast<int64_t>(blockIdx.x) * E + t];
#pragma unroll
    for (int v = 0; v < kScatterWaves; ++v) {
      base[v][t] = b;
      b += cnt[v][t];
    }
  }
  __syncthreads();
  const uint64_t below = (uint64_t(1) << lane) - 1;
#pragma unroll
  for (int i = 0; i < kScatterSteps; ++i) {
    const int s = p0 + 64 * i;
    if (s >= pend) break;
    const int p = s + lane;
    const int e = idv[i];
    const bool ok = e >= 0 && e < E;
    uint64_t m = __ballot(ok);
#pragma unroll 1
    for (int b = 0; b < nbits; ++b) {
      const bool bit = ok && ((e >> b) & 1);
      const uint64_t bb = __ballot(bit);
      m &= bit ? bb : ~bb;
    }
    // m: lanes holding the same expert (valid lanes only)
    int pos = 0;
    if (ok) pos = base[w][e] + __popcll(m & below);
    __builtin_amdgcn_wave_barrier();   // every lane has read base[w] for this step
    if (ok) {
      if (lane == 63 - __clzll(m)) base[w][e] += __popcll(m);   // the group's highest lane
      perm[pos] = p;
      inv_perm[p] = pos;
    } else if (p < pend) {
      inv_perm[p] = -1;                            // routed to an expert not in this call
    }
    __builtin_amdgcn_wave_barrier();
  }
}

__global__ __launch_bounds__(256) void gather_kernel(const uint4* __restrict__ x, const int32_t* __restrict__ perm,
                                                     const int32_t* __restrict__ rows_used, int P, int T, int k,
                                                     int64_t row_chunks, uint4* __restrict__ xp) {
  const int r = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (r >= P || r >= *rows_used) return;           // rows past offsets[E] do not exist
  const int lane = threadIdx.x & 63;
  int64_t t = perm[r] / k;
  t = t < 0 ? 0 : (t >= T ? T - 1 : t);   // rows left unwritten by invalid ids stay in bounds
  const uint4* src = x + t * row_chunks;
  uint4* dst = xp + static_cast<int64_t>(r) * row_chunks;
  for (int64_t c = lane; c < row_chunks; c += 64) dst[c] = src[c];
}

// All of histogram, scan and stable scatter in one workgroup, for at most
// kChunk pairs (small batches): one launch instead of three.
__global__ __launch_bounds__(256) void permute_small_kernel(const int32_t* __restrict__ ids, int P, int E, int nbits,
                                                            int32_t* __restrict__ counts,
                                                            int32_t* __restrict__ offsets,
                                                            int32_t* __restrict__ perm,
                                                            int32_t* __restrict__ inv_perm) {
  __shared__ int h[kMaxE];
  __shared__ int base[kMaxE];
  __shared__ int wsum[4];
  const int t = threadIdx.x;
  for (int e = t; e < E; e += 256) h[e] = 0;
  __syncthreads();
  for (int p = t; p < P; p += 256) {
    const int e = ids[p];
    if (e >= 0 && e < E) atomicAdd(&h[e], 1);
  }
  __syncthreads();
  // exclusive scan over experts, thread e owns expert e
  const int lane = t & 63, w = t >> 6;
  const int c = t < E ? h[t] : 0;
  int v = c;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int u = __shfl_up(v, o, 64);
    if (lane >= o) v += u;
  }
  if (lane == 63) wsum[w] = v;
  __syncthreads();
  int pre = 0;
  for (int i = 0; i < w; ++i) pre += wsum[i];
  const int excl = pre + v - c;
  if (t < E) {
    counts[t] = c;
    offsets[t] = excl;
    base[t] = excl;
  }
  if (t == E - 1) offsets[E] = excl + c;
  __syncthreads();
  if (w != 0) return;
  // stable scatter by the first wave, 64 pairs at a time in order, every id
  // loaded before the walk
  constexpr int kSteps = kChunk / 64;
  int idv[kSteps];
#pragma unroll
  for (int i = 0; i < kSteps; ++i) idv[i] = 64 * i + lane < P ? ids[64 * i + lane] : -1;
  const uint64_t below = (uint64_t(1) << lane) - 1;
#pragma unroll
  for (int i = 0; i < kSteps; ++i) {
    const int s0 = 64 * i;
    if (s0 >= P) break;
    const int p = s0 + lane;
    const int e = idv[i];
    const bool ok = e >= 0 && e < E;
    uint64_t m = __ballot(ok);
#pragma unroll 1
    for (int b = 0; b < nbits; ++b) {
      const bool bit = ok && ((e >> b) & 1);
      const uint64_t bb = __ballot(bit);
      m &= bit ? bb : ~bb;
    }
    int pos = 0;
    if (ok) pos = base[e] + __popcll(m & below);
    __builtin_amdgcn_wave_barrier();
    if (ok) {
      if (lane == 63 - __clzll(m)) base[e] += __popcll(m);
      perm[pos] = p;
      inv_perm[p] = pos;
    } else if (p < P) {
      inv_perm[p] = -1;                            // routed to an expert not in this call
    }
    __builtin_amdgcn_wave_barrier();
  }
}

__global__ void zero_kernel(int32_t* __restrict__ a, int n) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) a[i] = 0;
}

}  // namespace
}  // namespace moe

using namespace moe;

extern "C" size_t moe_permute_workspace_size(int64_t T, int32_t k, int32_t E) {
  if (T < 0 || k < 1 || E < 1 || E > kMaxE) return 0;
  return ws_bytes_for(T * k, E);
}

namespace moe {
namespace {

// The sort, with its per-chunk counts in a workspace of ws_bytes bytes
// (ws_given: there is one).  Shared by moe_permute (the caller's workspace)
// and moe_permute_noalloc (the library's static scratch).  `ws_of` yields
// the workspace's device address; it is called only once every check has
// passed, so a rejected call touches neither the workspace nor the GPU.
template <class WsOf>
moe_status permute_impl(const int32_t* topk_ids, const void* x, int64_t T, int64_t d, int32_t E, int32_t k,
                        moe_dtype dtype, int32_t* counts, int32_t* offsets, int32_t* perm, int32_t* inv_perm,
                        void* x_perm, size_t ws_bytes, bool ws_given, WsOf ws_of, void* stream) {
  // k may exceed E: with an expert-parallel share, the pairs of experts held
  // elsewhere carry ids outside [0, E)
  if (T < 0 || d < 0 || E < 1 || k < 1 || k > kMaxK) return MOE_ERR_INVALID_ARG;
  if (E > kMaxE) return MOE_ERR_UNSUPPORTED;
  if (!valid_dtype(dtype)) return MOE_ERR_INVALID_ARG;
  const int64_t P = T * k;
  if (P >= (int64_t(1) << 31)) return MOE_ERR_UNSUPPORTED;
  if (!counts || !offsets) return MOE_ERR_INVALID_ARG;
  if (x_perm && (d % 64 != 0)) return MOE_ERR_ALIGNMENT;
  if (x_perm && !x) return MOE_ERR_INVALID_ARG;
  if (x_perm && (!aligned16(x) || !aligned16(x_perm))) return MOE_ERR_ALIGNMENT;
  hipStream_t st = as_stream(stream);
  if (P == 0) {
    // a fill kernel rather than hipMemsetAsync, so the call can be captured in a graph
    hipLaunchKernelGGL(zero_kernel, dim3(1), dim3(kMaxE), 0, st, counts, E);
    hipLaunchKernelGGL(zero_kernel, dim3(2), dim3(kMaxE), 0, st, offsets, E + 1);
    return launch_status();
  }
  if (!topk_ids || !perm || !inv_perm) return MOE_ERR_INVALID_ARG;
  const size_t need = ws_bytes_for(P, E);
  if (!ws_given || ws_bytes < need) return MOE_ERR_WORKSPACE;
  int32_t* cc = nullptr;
  if (moe_status s = ws_of(cc); s != MOE_OK) return s;
  const int chunks = static_cast<int>(ceil_div(P, kChunk));
  int nbits = 0;
  while ((1 << nbits) < E) ++nbits;

  if (chunks == 1) {
    hipLaunchKernelGGL(permute_small_kernel, dim3(1), dim3(256), 0, st, topk_ids, static_cast<int>(P), E, nbits,
                       counts, offsets, perm, inv_perm);
  } else {
    hipLaunchKernelGGL(hist_kernel, dim3(chunks), dim3(256), 0, st, topk_ids, static_cast<int>(P), E, cc);
    hipLaunchKernelGGL(scan_kernel, dim3(1), dim3(256 * kScanParts), 0, st, cc, chunks, E, counts, offsets);
    hipLaunchKernelGGL(scatter_kernel, dim3(chunks), dim3(64 * kScatterWaves), 0, st, topk_ids, static_cast<int>(P), E, nbits,
                       cc, perm, inv_perm);
  }
  if (x_perm) {
    const int64_t row_chunks = d * elem_bytes(dtype) / 16;
    hipLaunchKernelGGL(gather_kernel, dim3(static_cast<unsigned>(ceil_div(P, 4))), dim3(256), 0, st,
                       static_cast<const uint4*>(x), perm, offsets + E, static_cast<int>(P), static_cast<int>(T),
                       k, row_chunks, static_cast<uint4*>(x_perm));
  }
  return launch_status();
}

// Scratch of moe_permute_noalloc: the per-chunk expert counts, in device
// memory the library owns (one copy per GPU, held until the process ends).
// Its name is a host-side stand-in: host code uses only the device address
// that hipGetSymbolAddress returns for the current device.
__device__ __align__(256) int32_t scratch[MOE_PERMUTE_SCRATCH_BYTES / sizeof(int32_t)];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
int32_t* g_scratch_ptr[kMaxDevices] = {};

// Device address of `scratch` on the current device, looked up once per
// device (with that device current) and kept.
moe_status scratch_on_current_device(int32_t*& out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return MOE_ERR_HIP;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return MOE_ERR_HIP;
    g_scratch_ptr[dev] = static_cast<int32_t*>(p);
  }
  out = g_scratch_ptr[dev];
  return MOE_OK;
}

}  // namespace
}  // namespace moe

extern "C" moe_status moe_permute(const int32_t* topk_ids, const void* x, int64_t T, int64_t d,
                                  int32_t E, int32_t k, moe_dtype dtype, int32_t* counts,
                                  int32_t* offsets, int32_t* perm, int32_t* inv_perm, void* x_perm,
                                  void* ws, size_t ws_bytes, void* stream) {
  return permute_impl(topk_ids, x, T, d, E, k, dtype, counts, offsets, perm, inv_perm, x_perm, ws_bytes,
                      ws != nullptr, [ws](int32_t*& cc) { cc = static_cast<int32_t*>(ws); return MOE_OK; },
                      stream);
}

extern "C" moe_status moe_permute_noalloc(const int32_t* topk_ids, const void* x, int64_t T, int64_t d,
                                          int32_t E, int32_t k, moe_dtype dtype, int32_t* counts,
                                          int32_t* offsets, int32_t* perm, int32_t* inv_perm, void* x_perm,
                                          void* stream) {
  return permute_impl(topk_ids, x, T, d, E, k, dtype, counts, offsets, perm, inv_perm, x_perm,
                      MOE_PERMUTE_SCRATCH_BYTES, true, scratch_on_current_device, stream);
}

// ---------------------------------------------------------------------------
// Expert-parallel share (article "Mixture of Experts (MoEs) in Transformers",
// section "Expert Parallelism"): a device holds the experts e_begin,
// e_begin + e_stride, ..., e_begin + (e_count - 1) e_stride (a contiguous
// block with stride 1); the router's global ids become local ids, and pairs
// whose expert lives elsewhere are masked (-1), so moe_permute gives them no
// row and moe_unpermute_combine adds nothing for them.
namespace moe {
namespace {
__global__ __launch_bounds__(256) void localize_kernel(const int32_t* __restrict__ ids, int64_t n, int e_begin,
                                                       int e_stride, int e_count, int32_t* __restrict__ out) {
  const int64_t i = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  if (i >= n) return;
  const int e = ids[i] - e_begin;
  const int j = e >= 0 ? e / e_stride : -1;
  out[i] = (e >= 0 && j * e_stride == e && j < e_count) ? j : -1;
}

moe_status localize(const int32_t* topk_ids, int64_t n, int32_t e_begin, int32_t e_stride, int32_t e_count,
                    int32_t* local_ids, void* stream) {
  if (n < 0 || e_begin < 0 || e_stride < 1 || e_count < 1) return MOE_ERR_INVALID_ARG;
  if (e_count > kMaxE) return MOE_ERR_UNSUPPORTED;
  if (n >= (int64_t(1) << 31)) return MOE_ERR_UNSUPPORTED;
  if (n == 0) return MOE_OK;
  if (!topk_ids || !local_ids) return MOE_ERR_INVALID_ARG;
  hipLaunchKernelGGL(localize_kernel, dim3(static_cast<unsigned>(ceil_div(n, 256))), dim3(256), 0, as_stream(stream),
                     topk_ids, n, e_begin, e_stride, e_count, local_ids);
  return launch_status();
}
// Any assignment of experts to the share: emap[e] is global expert e's
// local id, negative where another share holds it.  Router ids outside
// [0, E) and map entries outside [0, e_count) give -1 as well.
__global__ __launch_bounds__(256) void localize_map_kernel(const int32_t* __restrict__ ids, int64_t n,
                                                           const int32_t* __restrict__ emap, int E, int e_count,
                                                           int32_t* __restrict__ out) {
  const int64_t i = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  if (i >= n) return;
  const int e = ids[i];
  const int j = (e >= 0 && e < E) ? emap[e] : -1;
  out[i] = (j >= 0 && j < e_count) ? j : -1;
}

moe_status localize_map(const int32_t* topk_ids, int64_t n, const int32_t* expert_map, int32_t E,
                        int32_t e_count, int32_t* local_ids, void* stream) {
  if (n < 0 || E < 1 || e_count < 1) return MOE_ERR_INVALID_ARG;
  if (E > kMaxE || e_count > kMaxE) return MOE_ERR_UNSUPPORTED;
  if (n >= (int64_t(1) << 31)) return MOE_ERR_UNSUPPORTED;
  if (n == 0) return MOE_OK;
  if (!topk_ids || !expert_map || !local_ids) return MOE_ERR_INVALID_ARG;
  hipLaunchKernelGGL(localize_map_kernel, dim3(static_cast<unsigned>(ceil_div(n, 256))), dim3(256), 0,
                     as_stream(stream), topk_ids, n, expert_map, E, e_count, local_ids);
  return launch_status();
}
}  // namespace
}  // namespace moe

extern "C" moe_status moe_localize_ids(const int32_t* topk_ids, int64_t n, int32_t e_begin, int32_t e_count,
                                       int32_t* local_ids, void* stream) {
  return moe::localize(topk_ids, n, e_begin, 1, e_count, local_ids, stream);
}

extern "C" moe_status moe_localize_ids_strided(const int32_t* topk_ids, int64_t n, int32_t e_begin,
                                               int32_t e_stride, int32_t e_count, int32_t* local_ids,
                                               void* stream) {
  return moe::localize(topk_ids, n, e_begin, e_stride, e_count, local_ids, stream);
}

extern "C" moe_status moe_localize_ids_mapped(const int32_t* topk_ids, int64_t n, const int32_t* expert_map,
                                              int32_t num_experts, int32_t e_count, int32_t* local_ids,
                                              void* stream) {
  return moe::localize_map(topk_ids, n, expert_map, num_experts, e_count, local_ids, stream);
}
