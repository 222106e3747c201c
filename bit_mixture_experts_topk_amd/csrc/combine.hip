// gnf4_combine: out[t] = sum_j w[t, j] * Y[inv[t*k + j]] in float32, j ascending.
//
// A plain HBM-streaming kernel: each thread owns 4 consecutive columns of one
// token, reads the k routed rows with 16-byte loads and writes one float4.
// The top-k mixture is implied by the pages' MoE layers (Jordan Anderson,
// jordananderson-pages.pages.dev, section "grouped-nf4-gemm & experts-4bit",
// first bullet); its form here is the standard weighted sum.
#include "common.h"

namespace gnf4 {

constexpr int kCombineThreads = 256;

__global__ __launch_bounds__(kCombineThreads) void combine_kernel(
    const float *__restrict__ Y, const int32_t *__restrict__ inv, const float *__restrict__ w,
    int T, int k, int N, int nblk, float *__restrict__ out) {
  const int t = blockIdx.x / nblk;
  const int c4 = (blockIdx.x % nblk) * kCombineThreads + threadIdx.x;  // float4 column index
  const int lane = threadIdx.x & 63;
  // Lane j holds the routed row and weight of slot j (k <= 64): one load each
  // for the whole token, then every row load of a group of 8 slots is in
  // flight before the first product.
  int pj = -1;
  float wj = 0.f;
  if (lane < k) {
    pj = inv[(size_t)t * k + lane];
    wj = w[(size_t)t * k + lane];
  }
  const bool col_ok = c4 * 4 < N;
  f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
  for (int j0 = 0; j0 < k; j0 += 8) {
    f32x4_t y[8];
    int p[8];
    float wt[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int j = j0 + u;
      p[u] = __shfl(pj, j & 63, 64);
      wt[u] = __shfl(wj, j & 63, 64);
      if (j < k && p[u] >= 0 && col_ok)
        y[u] = *reinterpret_cast<const f32x4_t *>(Y + (size_t)p[u] * N + (size_t)c4 * 4);
      else
        y[u] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    }
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      if (j0 + u < k && p[u] >= 0) {        // dropped slots contribute nothing, j ascending
        acc[0] = __builtin_fmaf(wt[u], y[u][0], acc[0]);
        acc[1] = __builtin_fmaf(wt[u], y[u][1], acc[1]);
        acc[2] = __builtin_fmaf(wt[u], y[u][2], acc[2]);
        acc[3] = __builtin_fmaf(wt[u], y[u][3], acc[3]);
      }
    }
  }
  if (col_ok) *reinterpret_cast<f32x4_t *>(out + (size_t)t * N + (size_t)c4 * 4) = acc;
}

hipError_t launch_combine(const float *Y, const int32_t *inv, const float *w, int32_t T,
                          int32_t k, int32_t N, float *out, hipStream_t s) {
  if (T == 0) return hipSuccess;
  const int n4 = N / 4;
  const int nblk = (n4 + kCombineThreads - 1) / kCombineThreads;
  hipLaunchKernelGGL(combine_kernel, dim3((unsigned)T * nblk), dim3(kCombineThreads), 0, s, Y, inv,
                     w, T, k, N, nblk, out);
  return hipGetLastError();
}

}  // namespace gnf4
