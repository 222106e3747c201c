// gnf4_route: histogram, exclusive scan and stable counting-sort permutation
// of the flat top-k assignments, in one workgroup (one wave when T*k <= 64,
// else 1024 threads).
//
// The pages run the grouped GEMM as one launch for all active experts behind
// a router (Jordan Anderson, jordananderson-pages.pages.dev, section
// "grouped-nf4-gemm & experts-4bit", first bullet). The grouping is a
// counting sort: deterministic by construction, because the only atomics are
// order-independent integer additions (histogram, per-tile cursor updates)
// and each assignment's position is derived from ballots over lower lanes and
// per-wave counts of lower waves, never from atomic return values.
#include "common.h"

namespace gnf4 {

__device__ __forceinline__ int wave_inclusive_scan(int v, int lane) {
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    int u = __shfl_up(v, d, 64);
    if (lane >= d) v += u;
  }
  return v;
}

// THREADS = 1024 for large T*k; 64 (a single wave, no workgroup barriers
// needed for the scatter tiles) when T*k <= 64.
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

  // Histogram of valid ids; ids outside [0, E) only raise the flag. Eight
  // loads per thread are issued before their atomics, so the memory latency
  // is paid once per eight tiles rather than once per tile.
  constexpr int kHB = THREADS == 64 ? 1 : 8;
  for (int f0 = 0; f0 < n; f0 += THREADS * kHB) {
    int ev[kHB];
#pragma unroll
    for (int u = 0; u < kHB; ++u) {
      const int f = f0 + u * THREADS + tid;
      ev[u] = THREADS == 64 ? id0 : (f < n ? ids[f] : 0);
    }
#pragma unroll
    for (int u = 0; u < kHB; ++u) {
      if (f0 + u * THREADS + tid >= n) continue;
      if ((unsigned)ev[u] < (unsigned)E)
        atomicAdd(&cursor[ev[u]], 1);
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

  // Stable scatter, one tile of THREADS consecutive assignments at a time.
  // Within a wave, lanes holding the same expert are found by matching the id
  // bit by bit with ballots; the rank among them is the count of matching
  // lower lanes. Lower waves' counts for that expert come from wcnt.
  // The ids of the tile two ahead are loaded before a tile is processed.
  const uint64_t lower = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  int e_cur = THREADS == 64 ? id0 : (tid < n ? ids[tid] : -1);
  int e_nxt = THREADS == 64 ? -1 : (THREADS + tid < n ? ids[THREADS + tid] : -1);
  for (int base = 0; base < n; base += THREADS) {
    const int f = base + tid;
    const int e = e_cur;
    e_cur = e_nxt;
    if (THREADS > 64) e_nxt = f + 2 * THREADS < n ? ids[f + 2 * THREADS] : -1;
    const bool valid = (unsigned)e < (unsigned)E;
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
    } else if (f < n) {
      inv[f] = -1;
    }
    __syncthreads();
    if (valid && rank == 0) {
      atomicAdd(&cursor[e], tot);        // one leader per (wave, expert); waves add in any order
      if (kWaves > 1) wcnt[wave][e] = 0;
    }
    __syncthreads();
  }
  if (tid == 0) {
    n_active[0] = nact;
    bad[0] = sbad;
  }
}

hipError_t launch_route(const int32_t *ids, int32_t T, int32_t k, int32_t E, int32_t *counts,
                        int32_t *offsets, int32_t *perm, int32_t *inv, int32_t *active,
                        int32_t *n_active, int32_t *bad, hipStream_t s) {
  const int n = T * k;
  int nbits = 0;
  while ((1 << nbits) < E) ++nbits;
  if (n <= 64)
    hipLaunchKernelGGL(route_kernel<64>, dim3(1), dim3(64), 0, s, ids, n, E, nbits, counts,
                       offsets, perm, inv, active, n_active, bad);
  else
    hipLaunchKernelGGL(route_kernel<1024>, dim3(1), dim3(1024), 0, s, ids, n, E, nbits, counts,
                       offsets, perm, inv, active, n_active, bad);
  return hipGetLastError();
}

}  // namespace gnf4
