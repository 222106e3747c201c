// gnf4_route: histogram, exclusive scan and stable counting-sort permutation
// of the flat top-k assignments.
//
// The pages run the grouped GEMM as one launch for all active experts behind
// a router (Jordan Anderson, jordananderson-pages.pages.dev, section
// "grouped-nf4-gemm & experts-4bit", first bullet). The grouping is a
// counting sort: deterministic by construction, because the only atomics are
// order-independent integer additions (histograms, per-tile cursor updates)
// and each assignment's position is derived from ballots over lower lanes and
// per-wave counts of lower waves, never from atomic return values.
//
// Up to kRouteOneGroup assignments: one workgroup (one wave when T*k <= 64)
// does everything in one launch. Above that, three launches over chunks of
// consecutive assignments, with the caller's workspace between them:
//   route_count_kernel    one workgroup per chunk: the chunk's histogram
//   route_scan_kernel     one workgroup: per expert, the exclusive sum of its
//                         chunk counts (each chunk's first position for the
//                         expert), the totals, offsets and the active list
//   route_scatter_kernel  one workgroup per chunk: the stable scatter from
//                         those first positions
// Workspace (int32): chunk c's count, then first position, of expert e at
// c * E + e; the chunk's bad-id flag at nchunks * E + c.
#include <algorithm>
#include <mutex>

#include "common.h"

namespace gnf4 {

constexpr int kRouteThreads = 1024;
constexpr int kRouteOneGroup = 1024;     // assignments routed by one workgroup
constexpr int kRouteChunkMin = 1024;     // assignments per chunk (multiple of kRouteThreads)
constexpr int kRouteChunksMax = 256;     // chunks grow beyond kRouteChunkMin past this many

__device__ __forceinline__ int wave_inclusive_scan(int v, int lane) {
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    int u = __shfl_up(v, d, 64);
    if (lane >= d) v += u;
  }
  return v;
}

// Stable scatter of assignments [begin, end), tile by tile of THREADS:
// cursor[e] (LDS) holds expert e's next free position and advances by the
// tile's count; wcnt is LDS scratch of the per-wave counts within a tile
// (zero on entry, zero on exit). Within a wave, lanes holding the same expert
// are found by matching the id bit by bit with ballots; the rank among them
// is the count of matching lower lanes, and lower waves' counts for that
// expert come from wcnt. The ids of the tile two ahead are loaded before a
// tile is processed. id0 (THREADS == 64 only): this lane's id, read before.
template <int THREADS>
__device__ __forceinline__ void scatter_range(const int32_t *__restrict__ ids, int begin, int end,
                                              int E, int nbits, int *cursor,
                                              uint16_t (*wcnt)[GNF4_MAX_EXPERTS], int id0,
                                              int32_t *__restrict__ perm,
                                              int32_t *__restrict__ inv) {
  constexpr int kWaves = THREADS / 64;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const uint64_t lower = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  int e_cur = THREADS == 64 ? id0 : (begin + tid < end ? ids[begin + tid] : -1);
  int e_nxt = THREADS == 64 ? -1 : (begin + THREADS + tid < end ? ids[begin + THREADS + tid] : -1);
  for (int base = begin; base < end; base += THREADS) {
    const int f = base + tid;
    const int e = e_cur;
    e_cur = e_nxt;
    if (THREADS > 64) e_nxt = f + 2 * THREADS < end ? ids[f + 2 * THREADS] : -1;
    const bool valid = f < end && (unsigned)e < (unsigned)E;
    uint64_t match = __ballot(valid);
    for (int b = 0; b < nbits; ++b) {
      const bool bit = (e >> b) & 1;
      const uint64_t bm = __ballot(bit);
      match &= bit ? bm : ~bm;
    }
    const int rank = __popcll(match & lower);
    const int tot = __popcll(match);
    if (kWaves > 1) {
      if (valid && rank == 0) wcnt[wave][e] = (uint16_t)tot;
      __syncthreads();
    }
    if (valid) {
      int pos = cursor[e] + rank;
      for (int w = 0; w < wave; ++w) pos += wcnt[w][e];
      perm[pos] = f;
      inv[f] = pos;
    } else if (f < end) {
      inv[f] = -1;
    }
    __syncthreads();
    if (valid && rank == 0) {
      atomicAdd(&cursor[e], tot);        // one leader per (wave, expert); waves add in any order
      if (kWaves > 1) wcnt[wave][e] = 0;
    }
    __syncthreads();
  }
}

// THREADS = 1024 for up to kRouteOneGroup assignments; 64 (a single wave,
// no workgroup barriers needed for the scatter tiles) when T*k <= 64.
template <int THREADS>
__global__ __launch_bounds__(THREADS) void route_kernel(
    const int32_t *__restrict__ ids, int n, int E, int nbits, int32_t *__restrict__ counts,
    int32_t *__restrict__ offsets, int32_t *__restrict__ perm, int32_t *__restrict__ inv,
    int32_t *__restrict__ active, int32_t *__restrict__ n_active, int32_t *__restrict__ bad) {
  constexpr int kWaves = THREADS / 64;
  __shared__ int cursor[GNF4_MAX_EXPERTS];                       // histogram, then cursor
  __shared__ uint16_t wcnt[kWaves][GNF4_MAX_EXPERTS];            // per-wave counts in a tile
  __shared__ int wsum[kWaves], wact[kWaves];
  __shared__ int sbad, run_c, run_a;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  // With one wave all assignments fit one tile: read them once.
  const int id0 = (THREADS == 64 && tid < n) ? ids[tid] : -1;
  for (int e = tid; e < E; e += THREADS) {
    cursor[e] = 0;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) wcnt[w][e] = 0;
  }
  if (tid == 0) {
    sbad = 0;
    run_c = 0;
    run_a = 0;
  }
  __syncthreads();

  // Histogram of valid ids; ids outside [0, E) only raise the flag.
  for (int f0 = 0; f0 < n; f0 += THREADS) {
    const int f = f0 + tid;
    const int ev = THREADS == 64 ? id0 : (f < n ? ids[f] : 0);
    if (f < n) {
      if ((unsigned)ev < (unsigned)E)
        atomicAdd(&cursor[ev], 1);
      else
        sbad = 1;
    }
  }
  __syncthreads();

  // Exclusive scan of counts and the compacted active list, THREADS experts
  // at a time with running totals.
  for (int e0 = 0; e0 < E; e0 += THREADS) {
    const int e = e0 + tid;
    const int c = e < E ? cursor[e] : 0;
    const int a = c > 0 ? 1 : 0;
    const int ci = wave_inclusive_scan(c, lane);
    const int ai = wave_inclusive_scan(a, lane);
    if (lane == 63) {
      wsum[wave] = ci;
      wact[wave] = ai;
    }
    __syncthreads();
    int coff = run_c, aoff = run_a, tc = 0, ta = 0;
    for (int w = 0; w < kWaves; ++w) {
      if (w < wave) {
        coff += wsum[w];
        aoff += wact[w];
      }
      tc += wsum[w];
      ta += wact[w];
    }
    const int excl = coff + ci - c;
    if (e < E) {
      counts[e] = c;
      offsets[e] = excl;
      if (e == E - 1) offsets[E] = excl + c;
      if (a) active[aoff + ai - 1] = e;
    }
    __syncthreads();                     // everyone has read run_c / run_a / wsum
    if (e < E) cursor[e] = excl;
    if (tid == 0) {
      run_c += tc;
      run_a += ta;
    }
    __syncthreads();
  }
  const int total = run_c, nact = run_a;
  for (int e = nact + tid; e < E; e += THREADS) active[e] = -1;
  for (int p = total + tid; p < n; p += THREADS) perm[p] = -1;

  scatter_range<THREADS>(ids, 0, n, E, nbits, cursor, wcnt, id0, perm, inv);
  if (tid == 0) {
    n_active[0] = nact;
    bad[0] = sbad;
  }
}

// ---------------------------------------------------------- chunked route

// Histogram of chunk blockIdx.x ([c * chunk, min(n, (c + 1) * chunk))) to
// ws[c * E + e]; its bad-id flag to ws[nchunks * E + c]. Eight id loads per
// thread are issued before their LDS atomics.
__global__ __launch_bounds__(kRouteThreads) void route_count_kernel(const int32_t *__restrict__ ids,
                                                                    int n, int E, int chunk,
                                                                    int32_t *__restrict__ ws) {
  __shared__ int hist[GNF4_MAX_EXPERTS];
  __shared__ int sbad;
  const int tid = threadIdx.x, c = blockIdx.x;
  for (int e = tid; e < E; e += kRouteThreads) hist[e] = 0;
  if (tid == 0) sbad = 0;
  __syncthreads();
  const int begin = c * chunk, end = min(n, begin + chunk);
  constexpr int kHB = 8;
  for (int f0 = begin; f0 < end; f0 += kRouteThreads * kHB) {
    int ev[kHB];
#pragma unroll
    for (int u = 0; u < kHB; ++u) {
      const int f = f0 + u * kRouteThreads + tid;
      ev[u] = f < end ? ids[f] : 0;
    }
#pragma unroll
    for (int u = 0; u < kHB; ++u) {
      if (f0 + u * kRouteThreads + tid >= end) continue;
      if ((unsigned)ev[u] < (unsigned)E)
        atomicAdd(&hist[ev[u]], 1);
      else
        sbad = 1;
    }
  }
  __syncthreads();
  for (int e = tid; e < E; e += kRouteThreads) ws[(int64_t)c * E + e] = hist[e];
  if (tid == 0) ws[(int64_t)gridDim.x * E + c] = sbad;
}

// One workgroup: for each expert e (one per thread, E <= 1024), the chunk
// counts become the exclusive running sum over chunks plus offsets[e], i.e.
// the first position of chunk c's rows of expert e; then counts, offsets,
// the active list, n_active, the bad-id flag, and perm = -1 past the total.
__global__ __launch_bounds__(kRouteThreads) void route_scan_kernel(
    int n, int E, int nchunks, int32_t *__restrict__ ws, int32_t *__restrict__ counts,
    int32_t *__restrict__ offsets, int32_t *__restrict__ perm, int32_t *__restrict__ active,
    int32_t *__restrict__ n_active, int32_t *__restrict__ bad) {
  constexpr int kWaves = kRouteThreads / 64;
  __shared__ int wsum[kWaves], wact[kWaves];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int e = tid;
  // per-expert running sum over the chunks, eight loads in flight
  int c = 0;
  if (e < E) {
    constexpr int kB = 8;
    for (int c0 = 0; c0 < nchunks; c0 += kB) {
      int v[kB];
#pragma unroll
      for (int u = 0; u < kB; ++u) v[u] = c0 + u < nchunks ? ws[(int64_t)(c0 + u) * E + e] : 0;
#pragma unroll
      for (int u = 0; u < kB; ++u) {
        if (c0 + u < nchunks) ws[(int64_t)(c0 + u) * E + e] = c;
        c += v[u];
      }
    }
  }
  // any chunk saw a bad id
  int b = 0;
  for (int i = tid; i < nchunks; i += kRouteThreads) b |= ws[(int64_t)nchunks * E + i];
  const int anybad = __syncthreads_or(b);
  // exclusive scan of the counts over experts, and the active list
  const int a = c > 0 ? 1 : 0;
  const int ci = wave_inclusive_scan(c, lane);
  const int ai = wave_inclusive_scan(a, lane);
  if (lane == 63) {
    wsum[wave] = ci;
    wact[wave] = ai;
  }
  __syncthreads();
  int coff = 0, aoff = 0, total = 0, nact = 0;
  for (int w = 0; w < kWaves; ++w) {
    if (w < wave) {
      coff += wsum[w];
      aoff += wact[w];
    }
    total += wsum[w];
    nact += wact[w];
  }
  const int excl = coff + ci - c;
  if (e < E) {
    counts[e] = c;
    offsets[e] = excl;
    if (e == E - 1) offsets[E] = excl + c;
    if (a) active[aoff + ai - 1] = e;
    for (int i = 0; i < nchunks; ++i) ws[(int64_t)i * E + e] += excl;
  }
  for (int i = nact + tid; i < E; i += kRouteThreads) active[i] = -1;
  for (int p = total + tid; p < n; p += kRouteThreads) perm[p] = -1;
  if (tid == 0) {
    n_active[0] = nact;
    bad[0] = anybad ? 1 : 0;
  }
}

// Stable scatter of chunk blockIdx.x from the first positions the scan left
// in the workspace.
__global__ __launch_bounds__(kRouteThreads) void route_scatter_kernel(
    const int32_t *__restrict__ ids, int n, int E, int nbits, int chunk,
    const int32_t *__restrict__ ws, int32_t *__restrict__ perm, int32_t *__restrict__ inv) {
  constexpr int kWaves = kRouteThreads / 64;
  __shared__ int cursor[GNF4_MAX_EXPERTS];
  __shared__ uint16_t wcnt[kWaves][GNF4_MAX_EXPERTS];
  const int tid = threadIdx.x, c = blockIdx.x;
  for (int e = tid; e < E; e += kRouteThreads) {
    cursor[e] = ws[(int64_t)c * E + e];
#pragma unroll
    for (int w = 0; w < kWaves; ++w) wcnt[w][e] = 0;
  }
  __syncthreads();
  const int begin = c * chunk, end = min(n, begin + chunk);
  scatter_range<kRouteThreads>(ids, begin, end, E, nbits, cursor, wcnt, -1, perm, inv);
}

// Assignments per chunk: kRouteChunkMin, or more (whole tiles) so that there
// are at most about kRouteChunksMax chunks.
static int64_t route_chunk(int64_t n) {
  int64_t c = (n + kRouteChunksMax - 1) / kRouteChunksMax;
  c = (c + kRouteThreads - 1) / kRouteThreads * kRouteThreads;
  return std::max<int64_t>(c, kRouteChunkMin);
}

size_t route_workspace_bytes(int64_t n, int32_t E) {
  if (n <= kRouteOneGroup) return 0;
  const int64_t nchunks = (n + route_chunk(n) - 1) / route_chunk(n);
  const int64_t words = nchunks * ((int64_t)E + 1);
  return (size_t)((words * 4 + 255) / 256 * 256);
}

hipError_t launch_route(const int32_t *ids, int32_t T, int32_t k, int32_t E, int32_t *counts,
                        int32_t *offsets, int32_t *perm, int32_t *inv, int32_t *active,
                        int32_t *n_active, int32_t *bad, void *workspace, hipStream_t s) {
  const int n = T * k;
  int nbits = 0;
  while ((1 << nbits) < E) ++nbits;
  if (n <= 64) {
    hipLaunchKernelGGL(route_kernel<64>, dim3(1), dim3(64), 0, s, ids, n, E, nbits, counts,
                       offsets, perm, inv, active, n_active, bad);
    return hipGetLastError();
  }
  if (n <= kRouteOneGroup) {
    hipLaunchKernelGGL(route_kernel<kRouteThreads>, dim3(1), dim3(kRouteThreads), 0, s, ids, n, E,
                       nbits, counts, offsets, perm, inv, active, n_active, bad);
    return hipGetLastError();
  }
  const int chunk = (int)route_chunk(n);
  const int nchunks = (n + chunk - 1) / chunk;
  int32_t *ws = static_cast<int32_t *>(workspace);
  hipLaunchKernelGGL(route_count_kernel, dim3(nchunks), dim3(kRouteThreads), 0, s, ids, n, E, chunk,
                     ws);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(route_scan_kernel, dim3(1), dim3(kRouteThreads), 0, s, n, E, nchunks, ws,
                     counts, offsets, perm, active, n_active, bad);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(route_scatter_kernel, dim3(nchunks), dim3(kRouteThreads), 0, s, ids, n, E,
                     nbits, chunk, ws, perm, inv);
  return hipGetLastError();
}

// ------------------------------------------- route without caller memory

// The chunked route's workspace for callers that cannot allocate (code under
// graph capture, serving loops, harnesses that forbid hipMalloc): one
// file-scope array per device, held until the process ends. 1 MiB covers
// every route with E <= 1023 (at most 256 chunks of 4 * (E + 1) bytes) and
// E = 1024 up to 255 chunks of 1024 assignments.
constexpr size_t kRouteScratchBytes = (size_t)1 << 20;
static __device__ __align__(256) int32_t route_scratch[kRouteScratchBytes / 4];

size_t route_scratch_bytes() { return kRouteScratchBytes; }

// Device address of this device's route_scratch, resolved once per device
// with that device current (in host code the array's name is not a device
// address). NULL if the lookup fails.
void *route_scratch_ptr(hipError_t *err) {
  static std::mutex mu;
  static void *ptrs[64] = {nullptr};
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess || dev < 0 || dev >= 64) {
    *err = e != hipSuccess ? e : hipErrorInvalidDevice;
    return nullptr;
  }
  std::lock_guard<std::mutex> lock(mu);
  if (!ptrs[dev]) {
    void *p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(route_scratch));
    if (e != hipSuccess || !p) {
      *err = e != hipSuccess ? e : hipErrorInvalidSymbol;
      return nullptr;
    }
    ptrs[dev] = p;
  }
  *err = hipSuccess;
  return ptrs[dev];
}

}  // namespace gnf4
