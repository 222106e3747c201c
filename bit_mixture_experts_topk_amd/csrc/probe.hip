// gnf4_read_probe: a plain streaming read, the device's achievable HBM read
// rate against which the decode GEMV's packed-weight bandwidth is judged.
//
// The pages measure their own link and bus ceilings rather than assuming
// them (GitHub profile pjordanandrsn, NVMe-tier bullets; Jordan Anderson,
// jordananderson-pages.pages.dev, section "grouped-nf4-gemm & experts-4bit",
// demonstration paragraph: a run at a percentage of the measured link's
// ceiling). The same holds for HBM: the published 8 TB/s is not what a kernel
// that reads a few tens of MB once can reach, so the library ships the
// plainest such kernel. Every thread issues U non-temporal 16-byte loads
// before using any of them (grid-stride), folds the words with XOR, and
// stores only if the fold hits one constant, so the loads stay live without
// a store per thread. Over a buffer larger than the 256 MB Infinity Cache the
// same call evicts it.
#include <algorithm>

#include "common.h"

namespace gnf4 {

constexpr int kProbeThreads = 256;
constexpr int kProbeU = 8;
constexpr uint32_t kProbeMagic = 0x8f1bbcdcu;

__global__ __launch_bounds__(kProbeThreads) void read_probe_kernel(const uint4 *__restrict__ src,
                                                                    int64_t n16, uint32_t *sink) {
  typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));
  const int64_t stride = (int64_t)gridDim.x * kProbeThreads;
  int64_t i = (int64_t)blockIdx.x * kProbeThreads + threadIdx.x;
  uint32_t acc = 0;
  for (; i + (kProbeU - 1) * stride < n16; i += kProbeU * stride) {
    u32x4_t v[kProbeU];
#pragma unroll
    for (int u = 0; u < kProbeU; ++u)
      v[u] = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t *>(src + i + u * stride));
#pragma unroll
    for (int u = 0; u < kProbeU; ++u) acc ^= v[u][0] ^ v[u][1] ^ v[u][2] ^ v[u][3];
  }
  for (; i < n16; i += stride) {
    const u32x4_t v = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t *>(src + i));
    acc ^= v[0] ^ v[1] ^ v[2] ^ v[3];
  }
  if (acc == kProbeMagic) sink[0] = acc;
}

hipError_t launch_read_probe(const void *src, int64_t nbytes, int32_t workgroups, uint32_t *sink,
                             hipStream_t s) {
  const int64_t n16 = nbytes / 16;
  if (n16 == 0) return hipSuccess;
  int64_t wg = workgroups > 0 ? workgroups : 8LL * device_cu_count();
  wg = std::min<int64_t>(wg, (n16 + kProbeThreads - 1) / kProbeThreads);
  hipLaunchKernelGGL(read_probe_kernel, dim3((unsigned)wg), dim3(kProbeThreads), 0, s,
                     reinterpret_cast<const uint4 *>(src), n16, sink);
  return hipGetLastError();
}

}  // namespace gnf4
