// Expert streaming from host RAM: a residency cache of S expert slots in HBM
// in front of a layer whose packed experts live in pinned host memory.
//
// The pages run the fused kernel as the only expert compute while the 4-bit
// experts stream from pinned host memory over PCIe (Jordan Anderson,
// jordananderson-pages.pages.dev, section "grouped-nf4-gemm & experts-4bit",
// demonstration paragraph of the first bullet; same section, experts4bit-qlora
// bullets: layer-granular offload from pinned CPU memory, hot experts kept
// resident while the cold tail streams), and model the per-token time as the
// streamed bytes over the link's speed plus a fixed per-host cost. Here the
// residency is decided on the GPU, so a decode step needs no host round trip:
//
//  * cache_stage_kernel (one workgroup): marks the experts the step's ids
//    need; a needed expert already in a slot is a hit (its slot is stamped
//    with the step); the misses, in ascending expert order, take the slots
//    that no hit uses, empty slots first, then the least recently used, ties
//    to the lower slot (a bitonic sort of (age, slot) keys in LDS). It
//    updates the residency tables, lists the (expert, slot) copies and
//    rewrites the ids as slot ids, so the grouped GEMM runs on the S cached
//    experts exactly as on the resident layer.
//  * cache_fill_kernel: copies each listed expert's packed bytes (codes,
//    scales and, for NF4_DQ, its second-level scales) from host memory into
//    its slot; the GPU reads the pinned pages over the host link with 16-byte
//    loads, eight in flight per lane.
#include "common.h"

namespace gnf4 {

constexpr int kStageThreads = 1024;

// State words: [0] steps staged since the reset, [1, 1 + E) slot of expert e
// (-1: not resident), [1 + E, 1 + E + S) expert in slot s (-1: empty),
// [1 + E + S, 1 + E + 2S) the step that last used slot s (0: never).
__global__ __launch_bounds__(256) void cache_reset_kernel(int32_t *__restrict__ state, int E, int S) {
  const int n = 1 + E + 2 * S;
  for (int i = (int)(blockIdx.x * blockDim.x + threadIdx.x); i < n; i += (int)(gridDim.x * blockDim.x))
    state[i] = (i == 0 || i >= 1 + E + S) ? 0 : -1;
}

__global__ __launch_bounds__(kStageThreads) void cache_stage_kernel(
    const int32_t *__restrict__ ids, int n, int E, int S, int32_t *__restrict__ state,
    int32_t *__restrict__ slot_ids, int32_t *__restrict__ copies) {
  __shared__ int slot_of[GNF4_MAX_EXPERTS];    // the state, read once into LDS
  __shared__ int expert_of[GNF4_MAX_EXPERTS];
  __shared__ int last_used[GNF4_MAX_EXPERTS];
  __shared__ int need[GNF4_MAX_EXPERTS];       // expert needed by this step
  __shared__ int inuse[GNF4_MAX_EXPERTS];      // slot holds a hit
  __shared__ uint64_t key[GNF4_MAX_EXPERTS];   // eviction order of the free slots
  __shared__ int wtot[kStageThreads / 64];
  __shared__ int s_step;
  int32_t *g_slot_of = state + 1, *g_expert_of = state + 1 + E, *g_last_used = state + 1 + E + S;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;

  // One memory round trip: the whole state and this thread's first ids.
  constexpr int kIds = 4;                       // ids held per thread (more are read again)
  int idr[kIds];
#pragma unroll
  for (int r = 0; r < kIds; ++r) {
    const int i = tid + r * kStageThreads;
    idr[r] = i < n ? ids[i] : -1;
  }
  for (int i = tid; i < 1 + E + 2 * S; i += kStageThreads) {
    const int w = state[i];
    if (i == 0) s_step = w + 1;
    else if (i < 1 + E) slot_of[i - 1] = w;
    else if (i < 1 + E + S) expert_of[i - 1 - E] = w;
    else last_used[i - 1 - E - S] = w;
  }
  for (int e = tid; e < E; e += kStageThreads) need[e] = 0;
  for (int s = tid; s < S; s += kStageThreads) inuse[s] = 0;
  __syncthreads();
#pragma unroll
  for (int r = 0; r < kIds; ++r)
    if ((unsigned)idr[r] < (unsigned)E) need[idr[r]] = 1;
  for (int i = tid + kIds * kStageThreads; i < n; i += kStageThreads) {
    const int e = ids[i];
    if ((unsigned)e < (unsigned)E) need[e] = 1;
  }
  __syncthreads();
  const int step = s_step;

  // One expert per thread (E <= 1024). A slot value outside [0, S) counts
  // as not resident.
  const int e = tid;
  const bool needed = e < E && need[e];
  int cur = needed ? slot_of[e] : -1;
  if ((unsigned)cur >= (unsigned)S) cur = -1;
  const bool hit = cur >= 0, miss = needed && cur < 0;
  if (hit) inuse[cur] = 1;
  const uint64_t mb = __ballot(miss);
  const int mpre = __popcll(mb & (lane ? (~0ull >> (64 - lane)) : 0ull));
  if (lane == 0) wtot[wave] = __popcll(mb);
  __syncthreads();
  int m = mpre, M = 0;
#pragma unroll
  for (int w = 0; w < kStageThreads / 64; ++w) {
    if (w < wave) m += wtot[w];
    M += wtot[w];
  }

  // Eviction keys of the slots no hit uses: (age, slot), age 0 for an empty
  // slot and 1 + the last step otherwise; used slots and the padding sort last.
  int P = 2;
  while (P < S) P <<= 1;
  for (int s = tid; s < P; s += kStageThreads) {
    uint64_t kk = ~0ull;
    if (s < S && !inuse[s]) {
      const int ex = expert_of[s];
      const uint32_t age = (unsigned)ex < (unsigned)E ? (uint32_t)last_used[s] + 1u : 0u;
      kk = ((uint64_t)age << 32) | (uint32_t)s;
    }
    key[s] = kk;
  }
  __syncthreads();
  for (int kk = 2; kk <= P; kk <<= 1) {
    for (int j = kk >> 1; j > 0; j >>= 1) {
      for (int i = tid; i < P; i += kStageThreads) {
        const int ixj = i ^ j;
        if (ixj > i) {
          const uint64_t x = key[i], y = key[ixj];
          if ((x > y) == ((i & kk) == 0)) {
            key[i] = y;
            key[ixj] = x;
          }
        }
      }
      __syncthreads();
    }
  }

  // Miss m takes the m-th slot of the eviction order (there are enough when
  // S >= the step's distinct experts, which the host checks). The changed
  // words go to the state in HBM, the new slot of every needed expert to LDS
  // (need[] now holds it).
  int slot = cur;
  if (miss) {
    const uint64_t kk = m < P ? key[m] : ~0ull;
    slot = kk == ~0ull ? -1 : (int)(uint32_t)kk;
    if (slot >= 0) {
      const int old = expert_of[slot];
      if ((unsigned)old < (unsigned)E) g_slot_of[old] = -1;
      g_expert_of[slot] = e;
      g_slot_of[e] = slot;
      g_last_used[slot] = step;
    }
    copies[1 + 2 * m] = e;
    copies[2 + 2 * m] = slot;
  } else if (hit) {
    g_last_used[cur] = step;
  }
  __syncthreads();                              // every read of need[] done
  if (e < E) need[e] = slot;
  if (tid == 0) {
    state[0] = step;
    copies[0] = M;
  }
  __syncthreads();
#pragma unroll
  for (int r = 0; r < kIds; ++r) {
    const int i = tid + r * kStageThreads;
    if (i < n) slot_ids[i] = (unsigned)idr[r] < (unsigned)E ? need[idr[r]] : -1;
  }
  for (int i = tid + kIds * kStageThreads; i < n; i += kStageThreads) {
    const int id = ids[i];
    slot_ids[i] = (unsigned)id < (unsigned)E ? need[id] : -1;
  }
}

hipError_t launch_cache_reset(int32_t *state, int32_t E, int32_t S, hipStream_t s) {
  const int n = 1 + E + 2 * S;
  hipLaunchKernelGGL(cache_reset_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, state,
                     E, S);
  return hipGetLastError();
}

hipError_t launch_cache_stage(const int32_t *ids, int32_t n, int32_t E, int32_t S, int32_t *state,
                              int32_t *slot_ids, int32_t *copies, hipStream_t s) {
  hipLaunchKernelGGL(cache_stage_kernel, dim3(1), dim3(kStageThreads), 0, s, ids, n, E, S, state,
                     slot_ids, copies);
  return hipGetLastError();
}

// ---------------------------------------------------------------- fill

constexpr int kFillThreads = 256, kFillUnroll = 8;
constexpr int kFillUnits = kFillThreads * kFillUnroll;   // 16-byte units per workgroup

// Source unit u (16 bytes) of expert e / destination unit of slot s: the
// expert's bytes are its segments (codes, scales, scales2) one after the other.
__device__ __forceinline__ void fill_addr(const CacheFillArgs &f, int64_t u, int e, int s,
                                          const uint4 *&src, uint4 *&dst) {
  int g = 0;
  while (g + 1 < f.nseg && u >= f.seg_units[g]) {
    u -= f.seg_units[g];
    ++g;
  }
  src = reinterpret_cast<const uint4 *>(f.src[g]) + (int64_t)e * f.seg_units[g] + u;
  dst = reinterpret_cast<uint4 *>(f.dst[g]) + (int64_t)s * f.seg_units[g] + u;
}

__global__ __launch_bounds__(kFillThreads) void cache_fill_kernel(CacheFillArgs f) {
  const int ci = (int)(blockIdx.x / (unsigned)f.chunks);
  const int64_t c = (int64_t)(blockIdx.x - (unsigned)ci * (unsigned)f.chunks);
  if (ci >= f.copies[0]) return;
  const int e = f.copies[1 + 2 * ci], s = f.copies[2 + 2 * ci];
  if ((unsigned)e >= (unsigned)f.E || (unsigned)s >= (unsigned)f.S) return;
  const int64_t u0 = c * kFillUnits + threadIdx.x;
  uint4 v[kFillUnroll];
  uint4 *dst[kFillUnroll];
  // Units past the expert's end reload its last unit (no branch around the
  // loads) and are not stored.
#pragma unroll
  for (int r = 0; r < kFillUnroll; ++r) {
    const int64_t u = min(u0 + (int64_t)r * kFillThreads, f.units - 1);
    const uint4 *src;
    fill_addr(f, u, e, s, src, dst[r]);
    v[r] = *src;
  }
#pragma unroll
  for (int r = 0; r < kFillUnroll; ++r)
    if (u0 + (int64_t)r * kFillThreads < f.units) *dst[r] = v[r];
}

hipError_t launch_cache_fill(const CacheFillArgs &f, int32_t max_copies, hipStream_t s) {
  const int64_t grid = (int64_t)max_copies * f.chunks;
  if (grid <= 0) return hipSuccess;
  if (grid > 0x7fffffff) return hipErrorInvalidValue;
  hipLaunchKernelGGL(cache_fill_kernel, dim3((unsigned)grid), dim3(kFillThreads), 0, s, f);
  return hipGetLastError();
}

int64_t cache_fill_chunks(int64_t units) { return (units + kFillUnits - 1) / kFillUnits; }

}  // namespace gnf4
